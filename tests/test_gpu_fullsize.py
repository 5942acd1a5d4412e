"""GPU parity at the benchmark sizes, in the configuration bench.py times
(same inputs from workloads/, same entry points, same workspace): the library
computes every output at full size and the WHOLE output is compared with the
fp64 oracle, element by element (tests/_fullsize.py evaluates the oracle per
(sequence, query head) block on a thread pool).  Each test prints its raw max
|err|, the max |err| beyond the bf16 output rounding, the Frobenius-relative
error and the oracle's CPU time."""
import functools

import pytest
import torch

import flash_attention_kv_amd as F
from tests._fullsize import assert_bar, compare_decode, compare_prefill, compare_to_ref
from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_prefill(name):
    w = WORKLOADS[name]
    q, k, v, offs = make_prefill_inputs(w, device=DEV)
    offs_t = torch.from_numpy(offs).to(DEV) if offs is not None else None
    tq, sk = (w.T_q, w.S_kv) if offs is None else (q.shape[0], q.shape[0])
    dt = F.BF16 if w.dtype == "bf16" else F.F32
    need = F.ring_attn_workspace_bytes(tq, sk, w.h_q, w.h_kv, w.d, w.C, w.causal, w.n_seqs, offs is not None, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    o = F.ring_attn_fwd(q, k, v, C=w.C, causal=w.causal, seq_offsets=offs_t, n_seqs=w.n_seqs,
                        workspace=ws, window=w.window)
    torch.cuda.synchronize()
    return w, q.cpu(), k.cpu(), v.cpu(), o.cpu(), offs


@functools.lru_cache(maxsize=1)
def _gqa_ring_reference():
    """The fp64 oracle output of the gqa_ring workload (268 MB), computed once
    and shared by the three tests that run that workload through different
    entry points; returns (stats of ring_attn_fwd's output, reference)."""
    w, q, k, v, o, _ = _run_prefill("gqa_ring")
    return compare_prefill(o, q, k, v, causal=True, keep_ref=True)


def test_gqa_ring_fullsize():
    st, _ = _gqa_ring_reference()
    assert_bar(st, "bf16", "gqa_ring full output")


@pytest.mark.parametrize("name", ["dense_causal", "gqa_swa", "ring_tiny"])
def test_dense_prefill_fullsize(name):
    w, q, k, v, o, _ = _run_prefill(name)
    st = compare_prefill(o, q, k, v, causal=w.causal, n_seqs=w.n_seqs, window=w.window,
                         out_bf16=w.dtype == "bf16")
    assert_bar(st, w.dtype, f"{name} full output")


def test_jagged_prefill_fullsize():
    w, q, k, v, o, offs = _run_prefill("jagged")
    st = compare_prefill(o, q, k, v, causal=True, seq_offsets=offs)
    assert_bar(st, "bf16", "jagged full output")


def test_decode_fullsize():
    w = WORKLOADS["decode"]
    q, k, v = make_decode_inputs(w, device=DEV)
    ws = torch.empty(F.splitkv_decode_workspace_bytes(w.B, w.h_q, w.d, w.n_chunks), dtype=torch.uint8, device=DEV)
    o = F.splitkv_decode(q, k, v, n_chunks=w.n_chunks, workspace=ws)
    torch.cuda.synchronize()
    st = compare_decode(o.cpu(), q.cpu(), k.cpu(), v.cpu())
    assert_bar(st, "bf16", "decode full output")


def _ring_chunks(w):
    q, k, v, _ = make_prefill_inputs(w, device=DEV)
    n = w.S_kv // w.C
    qs = [q[r * n:(r + 1) * n] for r in range(w.C)]
    ks = [k[c * n:(c + 1) * n] for c in range(w.C)]
    vs = [v[c * n:(c + 1) * n] for c in range(w.C)]
    return q, k, v, qs, ks, vs, n


def test_ring_from_chunk_partials_fullsize():
    """The GQA ring at full size assembled from the chunk-level entry point,
    as the prefill page's ranks run it: rank r folds chunk (r + s) mod C into
    its running (m, l, O) at step s (attn_partial with accumulate), then
    divides by l.  Chunks wholly after the rank's queries are still passed and
    must leave the state unchanged.  The fp32 result is checked at the plain
    bar, over the whole output."""
    w = WORKLOADS["gqa_ring"]
    q, k, v, qs, ks, vs, n = _ring_chunks(w)
    outs = []
    for r in range(w.C):
        state = None
        for s in range(w.C):
            c = (r + s) % w.C
            state = F.attn_partial(qs[r], ks[c], vs[c], q_pos0=r * n, k_pos0=c * n, causal=True, state=state)
        m, l, o = state
        outs.append((o / l.unsqueeze(-1)).cpu())
    torch.cuda.synchronize()
    _, ref = _gqa_ring_reference()
    st = compare_to_ref(torch.cat(outs), ref, out_bf16=False)
    assert_bar(st, "bf16", "ring from attn_partial, full output")


def test_lse_merge_of_chunk_partials_fullsize():
    """The same ring as C separate chunk partials per rank (accumulate = 0)
    folded by one n-way lse_merge, rows = tokens x heads: parts of chunks
    after a rank's queries are empty (m = -inf, l = 0) and must weigh 0."""
    w = WORKLOADS["gqa_ring"]
    q, k, v, qs, ks, vs, n = _ring_chunks(w)
    rows = w.T_q * w.h_q
    m_parts = torch.empty(w.C, rows, dtype=torch.float32, device=DEV)
    l_parts = torch.empty_like(m_parts)
    o_parts = torch.empty(w.C, rows, w.d, dtype=torch.float32, device=DEV)
    for r in range(w.C):
        sl = slice(r * n * w.h_q, (r + 1) * n * w.h_q)
        for s in range(w.C):
            c = (r + s) % w.C
            m, l, o = F.attn_partial(qs[r], ks[c], vs[c], q_pos0=r * n, k_pos0=c * n, causal=True)
            m_parts[s, sl] = m.reshape(-1)
            l_parts[s, sl] = l.reshape(-1)
            o_parts[s, sl] = o.reshape(-1, w.d)
    out, lse = F.lse_merge(m_parts, l_parts, o_parts, out_dtype=torch.bfloat16, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    _, ref = _gqa_ring_reference()
    st = compare_to_ref(out.reshape(w.T_q, w.h_q, w.d).cpu(), ref, out_bf16=True)
    assert_bar(st, "bf16", "lse_merge of chunk partials, full output")

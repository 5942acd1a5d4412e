"""GPU parity at the benchmark sizes, in the configuration bench.py times
(same inputs from workloads/, same entry points, same workspace): every
output is computed by the library at full size, and a sample of output rows
-- first and last rows, rows at tile and chunk boundaries, rows of the
shortest and longest jagged sequences, and random ones -- is checked against
the fp64 oracle evaluated row by row from the definition."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import WORKLOADS, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample_rows(T, h_q, rng, extra=(), n_rand=40):
    toks = {0, T - 1, 63, 64, 127, 128, T // 2, T // 2 - 1, T // 8, T // 8 - 1} | set(extra)
    toks |= set(rng.integers(0, T, n_rand).tolist())
    toks = sorted(t for t in toks if 0 <= t < T)
    heads = rng.integers(0, h_q, len(toks))
    heads[0], heads[-1] = 0, h_q - 1
    return np.array(toks), heads


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


@pytest.mark.parametrize("name", ["gqa_ring", "dense_causal", "gqa_swa"])
def test_dense_prefill_fullsize_sampled(name):
    w, q, k, v, o, _ = _run_prefill(name)
    T = q.shape[0]
    rng = np.random.default_rng(123)
    chunk = w.S_kv // w.C
    bounds = [c * chunk + e for c in range(w.C) for e in (-1, 0)]
    bounds += [s * w.T_q + e for s in range(w.n_seqs) for e in (-1, 0)]
    toks, heads = _sample_rows(T, w.h_q, rng, extra=bounds)
    ref = oracle.attention_rows_ref(q, k, v, toks, heads, causal=w.causal, n_seqs=w.n_seqs, window=w.window)
    got = o.float().numpy()[toks, heads].astype(np.float64)
    check(got, ref, w.dtype, f"{name} sampled rows")
    assert torch.isfinite(o.float()).all()


def test_jagged_prefill_fullsize_sampled():
    w, q, k, v, o, offs = _run_prefill("jagged")
    T = q.shape[0]
    L = np.diff(offs)
    rng = np.random.default_rng(7)
    short, long_ = int(np.argmin(L)), int(np.argmax(L))
    extra = [offs[short], offs[short + 1] - 1, offs[long_], offs[long_ + 1] - 1, offs[long_] + 127,
             offs[long_] + 128, offs[-2], T - 1]
    toks, heads = _sample_rows(T, w.h_q, rng, extra=extra)
    ref = oracle.attention_rows_ref(q, k, v, toks, heads, causal=True, seq_offsets=offs)
    check(o.float().numpy()[toks, heads].astype(np.float64), ref, "bf16", "jagged sampled rows")
    assert torch.isfinite(o.float()).all()


def test_decode_fullsize_sampled():
    w = WORKLOADS["decode"]
    q, k, v = make_decode_inputs(w, device=DEV)
    ws = torch.empty(F.splitkv_decode_workspace_bytes(w.B, w.h_q, w.d, w.n_chunks), dtype=torch.uint8, device=DEV)
    o = F.splitkv_decode(q, k, v, n_chunks=w.n_chunks, workspace=ws).cpu()
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    rng = np.random.default_rng(3)
    picks = [(0, 0), (w.B - 1, w.h_q - 1)] + [(int(b), int(h)) for b, h in
                                              zip(rng.integers(0, w.B, 10), rng.integers(0, w.h_q, 10))]
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    got, ref = [], []
    for b, h in picks:
        got.append(o[b, h].float().numpy().astype(np.float64))
        ref.append(oracle.attention_rows_ref(qc[b:b + 1], kc[b], vc[b], [0], [h])[0])
    check(np.array(got), np.array(ref), "bf16", "decode sampled rows")


def _ring_chunks(w):
    q, k, v, _ = make_prefill_inputs(w, device=DEV)
    n = w.S_kv // w.C
    qs = [q[r * n:(r + 1) * n] for r in range(w.C)]
    ks = [k[c * n:(c + 1) * n] for c in range(w.C)]
    vs = [v[c * n:(c + 1) * n] for c in range(w.C)]
    return q, k, v, qs, ks, vs, n


def test_ring_from_chunk_partials_fullsize_sampled():
    """The GQA ring at full size assembled from the chunk-level entry point,
    as the prefill page's ranks run it: rank r folds chunk (r + s) mod C into
    its running (m, l, O) at step s (attn_partial with accumulate), then
    divides by l.  Chunks wholly after the rank's queries are still passed and
    must leave the state unchanged."""
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
    got_all = torch.cat(outs)
    assert torch.isfinite(got_all).all()
    rng = np.random.default_rng(11)
    toks, heads = _sample_rows(w.T_q, w.h_q, rng, extra=[c * n + e for c in range(w.C) for e in (-1, 0)])
    ref = oracle.attention_rows_ref(q.cpu(), k.cpu(), v.cpu(), toks, heads, causal=True)
    check(got_all.numpy()[toks, heads].astype(np.float64), ref, "bf16", "ring from attn_partial", out_bf16=False)


def test_lse_merge_of_chunk_partials_fullsize_sampled():
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
    out = out.reshape(w.T_q, w.h_q, w.d).cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(12)
    toks, heads = _sample_rows(w.T_q, w.h_q, rng, extra=[c * n + e for c in range(w.C) for e in (-1, 0)])
    ref = oracle.attention_rows_ref(q.cpu(), k.cpu(), v.cpu(), toks, heads, causal=True)
    check(out.float().numpy()[toks, heads].astype(np.float64), ref, "bf16", "lse_merge of chunk partials")

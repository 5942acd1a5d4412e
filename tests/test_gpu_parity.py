"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on
seeded inputs small enough for the oracle yet spanning several tiles, ragged
tails, GQA groupings, ring chunk counts, jagged batches and empty sequences;
plus the invariants that must hold bit for bit on the GPU (causal pruning =
masking, run-to-run determinism) and the integer worklist (bit-exact)."""
import json
import os

import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import WORKLOADS, make_prefill_inputs, randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qkv(Tq, Sk, h_q, h_kv, d, dtype, seed):
    q, k, v = randn([(Tq, h_q, d), (Sk, h_kv, d), (Sk, h_kv, d)], seed, dtype)
    return q, k, v


def _run_ring(q, k, v, **kw):
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return host(o)


def test_ring_tiny_f32_matches_oracle():
    w = WORKLOADS["ring_tiny"]
    q, k, v, _ = make_prefill_inputs(w)
    got = _run_ring(q, k, v, C=w.C, causal=w.causal)
    ref = oracle.ring_ref(q, k, v, w.C, causal=w.causal)
    check(got, ref, "f32", "ring_tiny")
    check(got, oracle.attention_ref(q, k, v), "f32", "ring_tiny vs monolithic")


PREFILL_CASES = [
    # T, h_q, h_kv, d, causal, C, n_seqs
    (1, 1, 1, 128, True, 1, 1),
    (37, 4, 1, 128, True, 1, 1),
    (130, 8, 2, 128, True, 2, 1),
    (256, 32, 8, 128, True, 8, 1),
    (300, 6, 3, 64, True, 3, 1),
    (255, 2, 1, 64, False, 5, 1),
    (200, 2, 2, 256, True, 4, 1),
    (129, 1, 1, 256, False, 1, 2),
    (96, 4, 4, 128, True, 1, 3),
    (64, 16, 1, 128, True, 4, 2),
    (513, 4, 2, 128, True, 1, 1),
]


@pytest.mark.parametrize("T,h_q,h_kv,d,causal,C,n_seqs", PREFILL_CASES)
def test_prefill_bf16_sweep(T, h_q, h_kv, d, causal, C, n_seqs):
    seed = T * 7 + h_q * 3 + d + C
    q, k, v = _qkv(n_seqs * T, n_seqs * T, h_q, h_kv, d, "bf16", seed)
    got = _run_ring(q, k, v, C=C, causal=causal, n_seqs=n_seqs)
    ref = oracle.attention_ref(q, k, v, causal=causal, n_seqs=n_seqs)
    check(got, ref, "bf16", f"bf16 T={T} h={h_q}/{h_kv} d={d} causal={causal} C={C}")


@pytest.mark.parametrize("T,S,h_q,h_kv,d,C", [(100, 40, 2, 1, 64, 2), (33, 256, 4, 2, 128, 4), (1, 96, 1, 1, 256, 3)])
def test_prefill_bf16_rectangular_noncausal(T, S, h_q, h_kv, d, C):
    q, k, v = _qkv(T, S, h_q, h_kv, d, "bf16", T + S)
    check(_run_ring(q, k, v, C=C), oracle.attention_ref(q, k, v), "bf16", "rect")


@pytest.mark.parametrize("T,h_q,h_kv,d,causal,C", [(130, 2, 1, 64, True, 2), (64, 1, 1, 128, False, 4),
                                                   (200, 4, 2, 256, True, 1), (33, 3, 3, 128, True, 3)])
def test_prefill_f32_sweep(T, h_q, h_kv, d, causal, C):
    q, k, v = _qkv(T, T, h_q, h_kv, d, "f32", T + d)
    got = _run_ring(q, k, v, C=C, causal=causal)
    check(got, oracle.attention_ref(q, k, v, causal=causal), "f32", "f32 sweep")


@pytest.mark.parametrize("T,h_q,causal,window", [(1024, 16, True, None), (128, 1, True, None),
                                                 (128, 1, False, None), (1024, 16, True, 300),
                                                 (96, 2, True, 40)])
def test_prefill_f32_fused_and_split(T, h_q, causal, window):
    """fp32 dense calls with 128 query tiles or more walk the ring in one
    workgroup per tile; smaller ones are split over their KV range (a partial
    per (tile, part), merged by lse_merge) and need a workspace.  Both paths
    against the oracle."""
    h_kv, d, C = 4 if h_q % 4 == 0 else 1, 64, 4
    split = F.ring_attn_workspace_bytes(T, T, h_q, h_kv, d, C, int(causal), 1, 0, F.F32) > 0
    assert split == (((T + 127) // 128) * h_q < 128)
    q, k, v = _qkv(T, T, h_q, h_kv, d, "f32", T + h_q)
    got = _run_ring(q, k, v, C=C, causal=causal, window=window)
    check(got, oracle.attention_ref(q, k, v, causal=causal, window=window), "f32",
          f"f32 {'split' if split else 'fused'} T={T} h={h_q}")


JAGGED = [[1, 0, 130, 64, 257, 2, 33], [0, 0, 5], [300], [128, 129, 127, 1, 1]]


@pytest.mark.parametrize("lens", JAGGED)
@pytest.mark.parametrize("heads,C", [((4, 4), 1), ((8, 2), 1), ((4, 1), 3)])
def test_jagged_bf16(lens, heads, C):
    h_q, h_kv = heads
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = _qkv(N, N, h_q, h_kv, 128, "bf16", N + h_q)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, causal=True,
                        seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.ring_ref(q, k, v, C, causal=True, seq_offsets=offs)
    check(host(o), ref, "bf16", f"jagged {lens} {heads} C={C}")


def test_jagged_f32():
    offs = seq_offsets_from_lengths([5, 200, 0, 64])
    N = int(offs[-1])
    q, k, v = _qkv(N, N, 2, 1, 64, "f32", 9)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    check(host(o), oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs), "f32", "jagged f32")


def test_worklist_bitexact_golden():
    g = json.load(open(os.path.join(GOLDEN, "worklist_small.json")))
    offs = torch.tensor(g["seq_offsets"], dtype=torch.int32, device=DEV)
    items, n = F.jagged_worklist(offs, g["seq_offsets"][-1], g["BQ"])
    n = int(n.item())
    np.testing.assert_array_equal(items[:n].cpu().numpy(), np.array(g["records"], dtype=np.int32))


@pytest.mark.parametrize("BQ", [32, 64, 128])
def test_worklist_bitexact_random(BQ):
    rng = np.random.default_rng(BQ)
    lens = rng.integers(0, 700, size=2000)
    lens[::37] = 0
    offs = seq_offsets_from_lengths(lens)
    items, n = F.jagged_worklist(torch.from_numpy(offs).to(DEV), int(offs[-1]), BQ)
    n = int(n.item())
    np.testing.assert_array_equal(items[:n].cpu().numpy(), oracle.worklist_array_ref(offs, BQ))


def test_worklist_rejects_bad_offsets():
    offs = torch.tensor([0, 5, 3, 10], dtype=torch.int32, device=DEV)   # decreasing
    items, n = F.jagged_worklist(offs, 10, 32)
    assert int(n.item()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_attn_partial_chain(dtype, causal):
    T, h_q, h_kv, d, C = 160, 4, 2, 128, 4
    q, k, v = _qkv(T, T, h_q, h_kv, d, dtype, 77 + causal)
    w = T // C
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    st, ref = None, None
    for step, c in enumerate((2, 0, 3, 1)):
        kc, vc = kd[c * w:(c + 1) * w].contiguous(), vd[c * w:(c + 1) * w].contiguous()
        st = F.attn_partial(qd, kc, vc, q_pos0=0, k_pos0=c * w, causal=causal, state=st)
        ref = oracle.attn_partial_ref(q, k[c * w:(c + 1) * w], v[c * w:(c + 1) * w], q_pos0=0,
                                      k_pos0=c * w, causal=causal, state=ref)
        torch.cuda.synchronize()
        m, l, o = (host(x) for x in st)
        fin = np.isfinite(ref.m)
        assert np.array_equal(np.isfinite(m), fin)
        np.testing.assert_allclose(m[fin], ref.m[fin], atol=1e-4, rtol=0)
        assert np.all(l[~fin] == 0) and np.all(o[~fin] == 0)
        np.testing.assert_allclose(l[fin], ref.l[fin], rtol=2e-2 if dtype == "bf16" else 1e-5)
        check(o[fin] / l[fin][:, None], ref.O[fin] / ref.l[fin][:, None], dtype, f"partial step {step}",
              out_bf16=False)
    check(host(st[2]) / host(st[1])[..., None], oracle.attention_ref(q, k, v, causal=causal), dtype,
          "partial chain vs monolithic", out_bf16=False)


def test_attn_partial_empty_chunk_writes_identity():
    q, k, v = _qkv(40, 8, 2, 1, 64, "bf16", 5)
    m, l, o = F.attn_partial(q.to(DEV), k.to(DEV), v.to(DEV), q_pos0=0, k_pos0=100, causal=True)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and not l.any() and not o.any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attn_partial_empty_chunk_tensors(dtype):
    """Zero-length K/V tensors (null data pointers): written alone the chunk
    gives the identity, merged into a running state it leaves the state as it
    was, bit for bit."""
    q, k, v = _qkv(40, 24, 4, 2, 128, dtype, 8)
    qd = q.to(DEV)
    ke, ve = k[:0].to(DEV), v[:0].to(DEV)
    m, l, o = F.attn_partial(qd, ke, ve, q_pos0=0, k_pos0=0, causal=False)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and not l.any() and not o.any()
    st = F.attn_partial(qd, k.to(DEV), v.to(DEV), q_pos0=30, k_pos0=0, causal=True)
    before = [t.clone() for t in st]
    st = F.attn_partial(qd, ke, ve, q_pos0=30, k_pos0=24, causal=True, state=st)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, st))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_lse_merge_matches_oracle(out):
    n, rows, d = 9, 50, 128
    rng = np.random.default_rng(3)
    m = rng.normal(size=(n, rows)) * 3
    m[2, :5] = -np.inf                         # empty parts
    l = np.where(np.isfinite(m), rng.uniform(0.5, 40, size=(n, rows)), 0.0)
    O = rng.normal(size=(n, rows, d)) * l[..., None]
    mt, lt, Ot = (torch.tensor(x, dtype=torch.float32, device=DEV) for x in (m, l, O))
    got, lse = F.lse_merge(mt, lt, Ot, out_dtype=torch.float32 if out == "f32" else torch.bfloat16,
                           return_lse=True)
    torch.cuda.synchronize()
    m32, l32, O32 = (host(x) for x in (mt, lt, Ot))
    for r in range(rows):
        ts = [oracle.Triplet(np.array([m32[c, r]]), np.array([l32[c, r]]), O32[c, r][None]) for c in range(n)]
        st = oracle.tree_merge_ref(ts)
        ref = oracle.finalize_ref(st)[0]
        g = host(got[r])
        if out == "f32":
            np.testing.assert_allclose(g, ref, rtol=2e-5, atol=1e-5)
        else:
            check(g, ref, "bf16", "merge bf16")
        assert abs(float(lse[r]) - (st.m[0] + np.log(st.l[0]))) < 1e-4


@pytest.mark.parametrize("B,h_q,h_kv,S,n_chunks", [(2, 8, 2, 1000, 7), (1, 64, 8, 4096, 16), (3, 4, 4, 77, 77),
                                                   (1, 32, 1, 300, 2), (2, 5, 5, 5, 4)])
def test_splitkv_decode_small(B, h_q, h_kv, S, n_chunks):
    d = 128
    q, k, v = randn([(B, h_q, d), (B, S, h_kv, d), (B, S, h_kv, d)], B * 100 + S, "bf16")
    o = F.splitkv_decode(q.to(DEV), k.to(DEV), v.to(DEV), n_chunks=n_chunks)
    torch.cuda.synchronize()
    ref = oracle.splitkv_decode_ref(q, k, v, n_chunks)
    check(host(o), ref, "bf16", f"decode B={B} h={h_q}/{h_kv} S={S} C={n_chunks}")


@pytest.mark.parametrize("d,heads,C", [(128, (8, 2), 2), (64, (2, 2), 1), (256, (4, 4), 3)])
def test_pruning_equals_masking_bitwise(d, heads, C, monkeypatch):
    h_q, h_kv = heads
    T = 384
    q, k, v = (x.to(DEV) for x in _qkv(T, T, h_q, h_kv, d, "bf16", d + C))
    a = F.ring_attn_fwd(q, k, v, C=C, causal=True)
    monkeypatch.setenv("FAKV_NO_PRUNE", "1")
    b = F.ring_attn_fwd(q, k, v, C=C, causal=True)
    monkeypatch.delenv("FAKV_NO_PRUNE")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_determinism_and_c_invariance():
    T, h_q, h_kv, d = 512, 8, 2, 128
    q, k, v = (x.to(DEV) for x in _qkv(T, T, h_q, h_kv, d, "bf16", 11))
    a = F.ring_attn_fwd(q, k, v, C=4, causal=True)
    b = F.ring_attn_fwd(q, k, v, C=4, causal=True)
    c1 = F.ring_attn_fwd(q, k, v, C=1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.attention_ref(host(q), host(k), host(v), causal=True)
    check(host(a), ref, "bf16", "C=4")
    check(host(c1), ref, "bf16", "C=1")
    assert float((a.float() - c1.float()).abs().max()) <= 1.5e-2


@pytest.mark.parametrize("heads", [(4, 4), (8, 2)])
def test_jagged_many_sequences(heads):
    """Over a thousand sequences (some empty): the device schedule spans several
    1024-wide scan chunks and every (tile, head group) must run exactly once."""
    h_q, h_kv = heads
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 300, size=1500)
    lens[::11] = 0
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = _qkv(N, N, h_q, h_kv, 128, "bf16", 23 + h_q)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    check(host(o), oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs), "bf16", f"jagged many {heads}")


@pytest.mark.parametrize("d,heads,C", [(64, (6, 2), 1), (64, (2, 2), 2), (256, (4, 2), 1), (256, (1, 1), 3)])
def test_jagged_bf16_head_dims(d, heads, C):
    """Jagged batches at the other head dims (the d = 64 and d = 256 tiles of
    the 8-wave jagged kernel): ragged lengths around the 256- and 128-row
    tiles, an empty sequence and a single token."""
    h_q, h_kv = heads
    lens = [257, 1, 0, 129, 512, 37]
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = _qkv(N, N, h_q, h_kv, d, "bf16", N + d + C)
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=C, causal=True,
                        seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    check(host(o), oracle.ring_ref(q, k, v, C, causal=True, seq_offsets=offs), "bf16", f"jagged d={d} {heads} C={C}")


@pytest.mark.parametrize("d,B,h_q,h_kv,S,n_chunks", [(64, 2, 16, 2, 1500, 9), (256, 1, 8, 8, 700, 5),
                                                      (256, 2, 32, 1, 333, 3)])
def test_splitkv_decode_head_dims(d, B, h_q, h_kv, S, n_chunks):
    q, k, v = randn([(B, h_q, d), (B, S, h_kv, d), (B, S, h_kv, d)], d + S, "bf16")
    o = F.splitkv_decode(q.to(DEV), k.to(DEV), v.to(DEV), n_chunks=n_chunks)
    torch.cuda.synchronize()
    check(host(o), oracle.splitkv_decode_ref(q, k, v, n_chunks), "bf16", f"decode d={d} B={B} h={h_q}/{h_kv}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("offs", [[0, 5, 3, 10], [0, 4, 9], [1, 4, 10]])
def test_jagged_bad_offsets_leave_output_untouched(dtype, offs):
    """Offsets that are not a prefix array of the T_q tokens (decreasing, last
    != total, first != 0) give an empty worklist: no kernel writes o."""
    N = 10
    q, k, v = _qkv(N, N, 2, 1, 64, dtype, 5)
    o = torch.full(q.shape, 7.0, dtype=q.dtype, device=DEV)
    F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True,
                    seq_offsets=torch.tensor(offs, dtype=torch.int32, device=DEV), out=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def test_binding_refuses_mismatched_out():
    """A caller-supplied output must match q exactly; the binding refuses it
    before anything is enqueued."""
    q, k, v = (t.to(DEV) for t in _qkv(64, 64, 4, 2, 128, "bf16", 1))
    for bad in (torch.empty(63, 4, 128, dtype=torch.bfloat16, device=DEV),
                torch.empty(64, 4, 128, dtype=torch.float32, device=DEV),
                torch.empty(4, 64, 128, dtype=torch.bfloat16, device=DEV).transpose(0, 1)):
        with pytest.raises(ValueError):
            F.ring_attn_fwd(q, k, v, causal=True, out=bad)
    qd = q[:2].clone()                                    # decode: (B=2, h_q=4, d)
    kc = torch.zeros(2, 64, 2, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        F.splitkv_decode(qd, kc, kc, n_chunks=2, out=torch.empty(2, 4, 64, dtype=torch.bfloat16, device=DEV))
    ws = F.splitkv_decode_workspace_bytes(2, 4, 128, 2)
    with pytest.raises(ValueError):                       # a workspace must be on the same device
        F.splitkv_decode(qd, kc, kc, n_chunks=2, workspace=torch.empty(ws, dtype=torch.uint8))

"""GPU parity on seeded random configurations.

The sweeps in test_gpu_parity.py pick their cases by hand; here a fixed list
of seeds draws configurations across the whole accepted space -- head dim,
GQA group (including groups that are not powers of two), dtype, dense or
jagged batch, ring chunk count, causal or not, sliding window, lengths that
are not tile multiples, empty sequences -- so that combinations nobody wrote
down still meet the oracle (the plain definition of softmax attention,
computed in fp64).  Each draw is reproducible from its seed alone."""
import os

import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# FAKV_EXTRA_SEEDS=N adds N more seeds (2000, 2001, ...) for a wider sweep
SEEDS = list(range(1000, 1032)) + list(range(2000, 2000 + int(os.environ.get("FAKV_EXTRA_SEEDS", "0"))))
DECODE_DRAWS = 16 + int(os.environ.get("FAKV_EXTRA_SEEDS", "0")) // 2


def _divisors(n, cap=8):
    return [c for c in range(1, cap + 1) if n % c == 0]


def draw(seed):
    """One configuration: a dict of everything the call and the oracle need."""
    r = np.random.RandomState(seed)
    d = int(r.choice([64, 128, 256]))
    g = int(r.choice([1, 2, 3, 4, 6, 8]))
    h_kv = int(r.choice([1, 2, 3])) if g <= 4 else 1
    dtype = "f32" if r.rand() < 0.25 else "bf16"
    jagged = bool(r.rand() < 0.4)
    cfg = dict(seed=seed, d=d, h_q=g * h_kv, h_kv=h_kv, dtype=dtype, jagged=jagged)
    if jagged:
        n = int(r.randint(1, 6))
        lens = [int(x) for x in r.randint(0, 420, size=n)]
        if r.rand() < 0.3:
            lens[int(r.randint(n))] = 0
        cfg.update(lens=lens, causal=bool(r.rand() < 0.8), C=int(r.choice([1, 1, 2, 3])))
    else:
        n_seqs = int(r.randint(1, 3))
        causal = bool(r.rand() < 0.7)
        T = int(r.randint(1, 520 // n_seqs))
        S = T if causal else int(r.randint(1, 520 // n_seqs))
        cfg.update(n_seqs=n_seqs, causal=causal, T=T, S=S, C=int(r.choice(_divisors(S))))
    cfg["window"] = int(r.randint(1, 300)) if cfg["causal"] and r.rand() < 0.35 else None
    return cfg


@pytest.mark.parametrize("seed", SEEDS)
def test_random_prefill_config(seed):
    c = draw(seed)
    tag = str(c)
    if c["jagged"]:
        offs = seq_offsets_from_lengths(c["lens"])
        N = int(offs[-1])
        q, k, v = randn([(N, c["h_q"], c["d"]), (N, c["h_kv"], c["d"]), (N, c["h_kv"], c["d"])], seed, c["dtype"])
        o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=c["C"], causal=c["causal"],
                            seq_offsets=torch.from_numpy(offs).to(DEV), window=c["window"])
        ref = oracle.attention_ref(q, k, v, causal=c["causal"], seq_offsets=offs, window=c["window"])
    else:
        n = c["n_seqs"]
        q, k, v = randn([(n * c["T"], c["h_q"], c["d"]), (n * c["S"], c["h_kv"], c["d"]),
                         (n * c["S"], c["h_kv"], c["d"])], seed, c["dtype"])
        o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), C=c["C"], causal=c["causal"], n_seqs=n,
                            window=c["window"])
        ref = oracle.attention_ref(q, k, v, causal=c["causal"], n_seqs=n, window=c["window"])
    torch.cuda.synchronize()
    check(host(o), ref, c["dtype"], tag)


def draw_decode(i):
    """One split-KV decode configuration: batch, GQA group (not only powers of
    two), head dim, cache length and chunk count (1 <= n_chunks <= S_kv;
    chunks of ceil(S / n) keys, so the last ones may be short or empty)."""
    r = np.random.RandomState(7000 + i)
    h_kv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 8]))
    S = int(r.randint(1, 3000))
    return dict(B=int(r.randint(1, 5)), h_q=g * h_kv, h_kv=h_kv, d=int(r.choice([64, 128, 256])), S=S,
                n_chunks=int(r.randint(1, min(70, S) + 1)))


@pytest.mark.parametrize("i", range(DECODE_DRAWS))
def test_random_decode_config(i):
    c = draw_decode(i)
    q, k, v = randn([(c["B"], c["h_q"], c["d"]), (c["B"], c["S"], c["h_kv"], c["d"]),
                     (c["B"], c["S"], c["h_kv"], c["d"])], 7000 + i, "bf16")
    o = F.splitkv_decode(q.to(DEV), k.to(DEV), v.to(DEV), n_chunks=c["n_chunks"])
    torch.cuda.synchronize()
    check(host(o), oracle.splitkv_decode_ref(q, k, v, c["n_chunks"]), "bf16", str(c))


PARTIAL_DRAWS = 12 + int(os.environ.get("FAKV_EXTRA_SEEDS", "0")) // 2


@pytest.mark.parametrize("i", range(PARTIAL_DRAWS))
def test_random_partial_chain(i):
    """A chain of attn_partial calls over KV chunks of random sizes (empty ones
    included) at random query and key positions, the first written and the
    rest merged into the running state, against the same chain in the oracle
    (the prefill page's ring step with explicit positions)."""
    r = np.random.RandomState(9000 + i)
    d = int(r.choice([64, 128, 256]))
    g = int(r.choice([1, 2, 3, 4, 8]))
    h_kv = int(r.choice([1, 2]))
    h_q = g * h_kv
    dtype = "f32" if r.rand() < 0.3 else "bf16"
    T, q_pos0, causal = int(r.randint(1, 300)), int(r.randint(0, 400)), bool(r.rand() < 0.6)
    sizes = [int(x) for x in r.randint(0, 250, size=int(r.randint(1, 5)))]
    k_pos = int(r.randint(0, 300))
    tag = f"d={d} h={h_q}/{h_kv} {dtype} T={T} q_pos0={q_pos0} causal={causal} chunks={sizes} k_pos0={k_pos}"
    q, = randn([(T, h_q, d)], 9000 + i, dtype)
    st, ref = None, None
    for c, S in enumerate(sizes):
        k, v = randn([(S, h_kv, d), (S, h_kv, d)], 9500 + 7 * i + c, dtype)
        st = F.attn_partial(q.to(DEV), k.to(DEV), v.to(DEV), q_pos0=q_pos0, k_pos0=k_pos, causal=causal, state=st)
        ref = oracle.attn_partial_ref(q, k, v, q_pos0=q_pos0, k_pos0=k_pos, causal=causal, state=ref)
        k_pos += S
    torch.cuda.synchronize()
    m, l, o = (host(x) for x in st)
    fin = np.isfinite(ref.m)
    assert np.array_equal(np.isfinite(m), fin), tag
    assert np.all(l[~fin] == 0) and np.all(o[~fin] == 0), tag
    if fin.any():
        np.testing.assert_allclose(m[fin], ref.m[fin], atol=1e-4, rtol=0, err_msg=tag)
        np.testing.assert_allclose(l[fin], ref.l[fin], rtol=2e-2 if dtype == "bf16" else 1e-5, err_msg=tag)
        check(o[fin] / l[fin][:, None], ref.O[fin] / ref.l[fin][:, None], dtype, tag, out_bf16=False)


def test_draws_cover_the_space():
    """The fixed seeds reach every head dim, both dtypes, both batch kinds,
    windows, ring chunking and non-power-of-two groups."""
    cs = [draw(s) for s in SEEDS]
    assert {c["d"] for c in cs} == {64, 128, 256}
    assert {c["dtype"] for c in cs} == {"bf16", "f32"}
    assert any(c["jagged"] for c in cs) and not all(c["jagged"] for c in cs)
    assert any(c["window"] for c in cs)
    assert any(c["C"] > 1 for c in cs)
    assert any((c["h_q"] // c["h_kv"]) in (3, 6) for c in cs)
    assert any(c["jagged"] and 0 in c["lens"] for c in cs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_empty_jagged_batch(dtype):
    """Sequences that are all empty: a valid call with nothing to compute (no
    workspace, empty tensors with null data pointers)."""
    offs = torch.zeros(4, dtype=torch.int32, device=DEV)
    t = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.empty(0, 8, 128, dtype=t, device=DEV)
    k = torch.empty(0, 2, 128, dtype=t, device=DEV)
    o = F.ring_attn_fwd(q, k, k, causal=True, seq_offsets=offs)
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 128)

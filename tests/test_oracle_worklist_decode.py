"""Pins of the oracle's worklist, split-KV decode, fan-out simulator and work counts."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import Triplet
from workloads import jagged_lengths, seq_offsets_from_lengths, WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_worklist_hand_fixture():
    g = json.load(open(os.path.join(GOLDEN, "worklist_small.json")))
    a = oracle.worklist_array_ref(g["seq_offsets"], g["BQ"])
    np.testing.assert_array_equal(a, np.array(g["records"], dtype=np.int32))


@pytest.mark.parametrize("BQ", [1, 32, 128])
def test_worklist_covers_every_query_once(BQ):
    lens = jagged_lengths(50, 0, 300, seed=3)
    offs = seq_offsets_from_lengths(lens)
    items = oracle.worklist_ref(offs, BQ)
    hit = np.zeros(int(offs[-1]), int)
    for it in items:
        assert it.range_start == offs[it.seq] and it.range_len == lens[it.seq]
        assert 1 <= it.tile_extent <= BQ and it.tile_start == offs[it.seq] + it.tile * BQ
        assert it.compute_end == it.tile_start + it.tile_extent <= it.range_start + it.range_len
        hit[it.tile_start:it.tile_start + it.tile_extent] += 1
    assert np.all(hit == 1)
    keys = [(-it.tile, it.seq) for it in items]
    assert keys == sorted(keys)
    assert len(items) == int(sum(-(-int(L) // BQ) for L in lens))


@pytest.mark.parametrize("order", ["tree", "linear", "chain"])
@pytest.mark.parametrize("n_chunks", [1, 3, 8])
def test_splitkv_decode_equals_monolithic(order, n_chunks):
    B, h_q, h_kv, d, S = 2, 8, 2, 4, 29
    q, k, v = _rand((B, h_q, d), 1), _rand((B, S, h_kv, d), 2), _rand((B, S, h_kv, d), 3)
    got = oracle.splitkv_decode_ref(q, k, v, n_chunks, order=order, rank=n_chunks // 2)
    for b in range(B):
        ref = oracle.attention_ref(q[b][None], k[b], v[b])[0]
        np.testing.assert_allclose(got[b], ref, rtol=1e-12, atol=1e-13)


def test_decode_empty_chunks():
    B, h_q, d, S = 1, 2, 4, 5
    q, k, v = _rand((B, h_q, d), 4), _rand((B, S, 1, d), 5), _rand((B, S, 1, d), 6)
    m, l, O = oracle.decode_partials_ref(q, k, v, 8)   # width 1: chunks 5..7 empty
    assert np.all(m[0, :, 5:] == -np.inf) and not l[0, :, 5:].any()
    np.testing.assert_allclose(oracle.splitkv_decode_ref(q, k, v, 8)[0],
                               oracle.attention_ref(q[0][None], k[0], v[0])[0], rtol=1e-12)


def test_fanout_hand_schedule():
    g = json.load(open(os.path.join(GOLDEN, "fanout_arrivals_n4.json")))
    n = g["n"]
    ts = [Triplet(np.array([float(r)]), np.array([1.0]), np.array([[float(r)]])) for r in range(n)]
    _, log = oracle.fanout_simulate(ts)
    assert [[list(x) for x in lg] for lg in log] == g["log"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 16])
def test_fanout_exactly_once_and_replicated(n):
    d = 4
    q, k, v = _rand((1, d), n), _rand((3 * n, d), n + 1), _rand((3 * n, d), n + 2)
    ts = [oracle.partial_ref(q, k[3 * r:3 * r + 3], v[3 * r:3 * r + 3], np.ones((1, 3), bool), 0.5)
          for r in range(n)]
    finals, log = oracle.fanout_simulate(ts)
    ref = oracle.attention_ref(q[None], k[:, None], v[:, None])[0]
    for r in range(n):
        origins = [o for _, o in log[r]]
        assert sorted(origins + [r]) == list(range(n))          # every origin exactly once
        assert all(s == abs(o - r) for s, o in log[r])            # arrives at step |i - j|
        assert [r] + origins == oracle.fanout_order(r, n)
        np.testing.assert_allclose(oracle.finalize_ref(finals[r]), ref, rtol=1e-12, atol=1e-13)


def test_fanout_detects_dropped_message():
    ts = [Triplet(np.array([0.0]), np.array([1.0]), np.array([[1.0]])) for _ in range(4)]

    def dropping_merge(a, b, _n=[0]):
        _n[0] += 1
        return a if _n[0] == 3 else oracle.merge_ref(a, b)
    finals, _ = oracle.fanout_simulate(ts, merge=dropping_merge)
    ls = [float(f.l[0]) for f in finals]
    assert ls.count(4.0) == 3 and 3.0 in ls


def test_counts_closed_forms_and_brute_force():
    import oracle
    for L in (1, 2, 7, 64):
        assert oracle.causal_pairs(L) == int(np.tril(np.ones((L, L))).sum())
    lens = [3, 0, 5]
    offs = [0, 3, 3, 8]
    assert oracle.prefill_pairs(8, 8, causal=True, seq_offsets=offs) == 6 + 0 + 15
    assert oracle.prefill_pairs(8, 8, causal=False, seq_offsets=offs) == 9 + 25
    assert oracle.prefill_pairs(8, 16, causal=False, n_seqs=2) == 2 * 4 * 8
    assert oracle.useful_flops_prefill(2, 8, 10) == 4 * 8 * 2 * 10
    assert oracle.decode_bytes(1, 2, 1, 4, 10) == 2 * 10 * 4 * 2 + 2 * 2 * 4 * 2


def test_decode_counts_brute_force():
    """decode_flops and decode_bytes against an enumeration: every (sequence,
    query head, cached key) pair costs d multiply-adds for its score and d for
    its value product (2 FLOP each); every K and V element of the cache is
    read once and every q and o element moved once."""
    import oracle
    for (B, h_q, h_kv, d, S) in [(1, 1, 1, 1, 1), (2, 4, 2, 3, 5), (3, 6, 3, 2, 7)]:
        flops = 0
        for _b in range(B):
            for _h in range(h_q):
                for _j in range(S):
                    flops += 2 * d      # score: d multiplies + d adds
                    flops += 2 * d      # value: d multiplies + d adds
        assert oracle.decode_flops(B, h_q, d, S) == flops
        # one query per sequence, every cached key admissible: the prefill count
        pairs = oracle.prefill_pairs(B, B * S, causal=False, n_seqs=B)
        assert oracle.decode_flops(B, h_q, d, S) == oracle.useful_flops_prefill(h_q, d, pairs)
        elems = sum(1 for _t in ("k", "v") for _b in range(B) for _j in range(S) for _h in range(h_kv)
                    for _x in range(d))
        elems += sum(1 for _t in ("q", "o") for _b in range(B) for _h in range(h_q) for _x in range(d))
        assert oracle.decode_bytes(B, h_q, h_kv, d, S) == 2 * elems


def test_workload_sizes():
    w = WORKLOADS["jagged"]
    offs = seq_offsets_from_lengths(jagged_lengths(w.n_seqs))
    assert int(offs[-1]) == 1240379
    pairs = oracle.prefill_pairs(0, 0, causal=True, seq_offsets=offs)
    assert pairs == 856208948
    assert oracle.useful_flops_prefill(4, 128, pairs) == 4 * 128 * 4 * 856208948
    g = WORKLOADS["gqa_ring"]
    assert oracle.useful_flops_prefill(32, 128, oracle.causal_pairs(8192)) == 549822922752
    dc = WORKLOADS["dense_causal"]
    assert oracle.useful_flops_prefill(32, 256, 8 * oracle.causal_pairs(4096)) == 2199560126464
    dw = WORKLOADS["decode"]
    assert oracle.decode_bytes(8, 64, 8, 128, 131072) == 4294967296 + 262144

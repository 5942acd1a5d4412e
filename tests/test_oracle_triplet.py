"""Pins of the oracle's partial / merge / ring / dependent-bound functions:
brute-force triplets, hand fixtures, merge algebra, ring = monolithic, chunk
order invariance, and pruning = masking (bitwise)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import Triplet
from tests._brute import brute_triplet

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _t(m, l, O):
    return Triplet(np.array([m], float), np.array([l], float), np.array([O], float))


def test_partial_brute_force():
    d, n = 3, 6
    q, kk, vv = _rand((4, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    allowed = np.array([[1, 1, 0, 1, 0, 0], [0, 0, 0, 0, 0, 0], [1, 1, 1, 1, 1, 1], [0, 0, 0, 0, 0, 1]], bool)
    t = oracle.partial_ref(q, kk, vv, allowed, 0.5)
    for r in range(4):
        m, l, O = brute_triplet(q[r].tolist(), kk.tolist(), vv.tolist(), allowed[r].tolist(), 0.5)
        assert t.m[r] == m or abs(t.m[r] - m) < 1e-14
        assert abs(t.l[r] - l) < 1e-13
        np.testing.assert_allclose(t.O[r], O, rtol=1e-13, atol=1e-14)
    assert t.m[1] == -np.inf and t.l[1] == 0 and not t.O[1].any()


def test_merge_fixtures():
    data = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    for c in data["merge_cases"]:
        a = _t(float(c["a"]["m"]), c["a"]["l"], c["a"]["O"])
        b = _t(float(c["b"]["m"]), c["b"]["l"], c["b"]["O"])
        for x, y in ((a, b), (b, a)):
            r = oracle.merge_ref(x, y)
            assert abs(r.m[0] - c["expect"]["m"]) < 1e-15, c["name"]
            assert abs(r.l[0] - c["expect"]["l"]) < 1e-15, c["name"]
            np.testing.assert_allclose(r.O[0], c["expect"]["O"], rtol=1e-15)
            np.testing.assert_allclose(oracle.finalize_ref(r)[0], c["expect"]["final"], rtol=1e-15)


def test_merge_identity_commutative_associative():
    d = 5
    ts = [oracle.partial_ref(_rand((3, d), s), _rand((4, d), s + 1), _rand((4, d), s + 2),
                             np.ones((3, 4), bool), 0.7) for s in (10, 20, 30)]
    I = oracle.identity_triplet(3, d)
    for t in ts:
        for r in (oracle.merge_ref(t, I), oracle.merge_ref(I, t)):
            assert np.array_equal(r.m, t.m) and np.array_equal(r.l, t.l) and np.array_equal(r.O, t.O)
    II = oracle.merge_ref(I, I)
    assert np.all(II.m == -np.inf) and not II.l.any() and not II.O.any()
    a, b, c = ts
    ab, ba = oracle.merge_ref(a, b), oracle.merge_ref(b, a)
    np.testing.assert_allclose(ab.O, ba.O, rtol=1e-15); np.testing.assert_allclose(ab.l, ba.l, rtol=1e-15)
    l1 = oracle.merge_ref(oracle.merge_ref(a, b), c)
    l2 = oracle.merge_ref(a, oracle.merge_ref(b, c))
    np.testing.assert_allclose(l1.O, l2.O, rtol=1e-13); np.testing.assert_allclose(l1.l, l2.l, rtol=1e-13)
    assert np.array_equal(l1.m, l2.m)


@pytest.mark.parametrize("C", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2)])
def test_ring_equals_monolithic(C, causal, heads):
    h_q, h_kv = heads
    T, d = 48, 8
    q, k, v = _rand((T, h_q, d), C), _rand((T, h_kv, d), C + 1), _rand((T, h_kv, d), C + 2)
    ref = oracle.attention_ref(q, k, v, causal=causal)
    np.testing.assert_allclose(oracle.ring_ref(q, k, v, C, causal=causal), ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.ring_ref(q, k, v, C, causal=causal, block_k=5), ref, rtol=1e-12, atol=1e-13)


def test_ring_rectangular_and_dense_batch():
    q, k, v = _rand((16, 2, 4), 1), _rand((64, 1, 4), 2), _rand((64, 1, 4), 3)
    np.testing.assert_allclose(oracle.ring_ref(q, k, v, 4), oracle.attention_ref(q, k, v), rtol=1e-12)
    q, k, v = _rand((3 * 24, 2, 4), 4), _rand((3 * 24, 2, 4), 5), _rand((3 * 24, 2, 4), 6)
    np.testing.assert_allclose(oracle.ring_ref(q, k, v, 4, causal=True, n_seqs=3),
                               oracle.attention_ref(q, k, v, causal=True, n_seqs=3), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 2, 3, 5])
def test_ring_jagged(C):
    lens = [1, 0, 7, 12, 64, 3]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(offs[-1])
    q, k, v = _rand((N, 2, 4), 7), _rand((N, 1, 4), 8), _rand((N, 1, 4), 9)
    ref = oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs)
    got = oracle.ring_ref(q, k, v, C, causal=True, seq_offsets=offs, block_k=4)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_c1_is_single_partial():
    q, k, v = _rand((10, 1, 6), 11), _rand((10, 1, 6), 12), _rand((10, 1, 6), 13)
    t = oracle.partial_ref(q[:, 0], k[:, 0], v[:, 0], np.tril(np.ones((10, 10), bool)), 1 / math.sqrt(6))
    np.testing.assert_allclose(oracle.finalize_ref(t), oracle.attention_ref(q, k, v, causal=True)[:, 0], rtol=1e-13)
    o, m, l = oracle.ring_ref(q, k, v, 1, causal=True, return_triplet=True)
    np.testing.assert_array_equal(m[:, 0], t.m)


@pytest.mark.parametrize("C", [2, 3, 4, 5])
def test_chunk_order_invariance_all_permutations(C):
    T, d = 20, 4
    S = 4 * C
    q, k, v = _rand((T, 1, d), 20 + C), _rand((S, 1, d), 21 + C), _rand((S, 1, d), 22 + C)
    ref = oracle.attention_ref(q, k, v)[:, 0]
    w = S // C
    parts = [oracle.partial_ref(q[:, 0], k[c * w:(c + 1) * w, 0], v[c * w:(c + 1) * w, 0],
                                np.ones((T, w), bool), 0.5) for c in range(C)]
    for perm in itertools.permutations(range(C)):
        st = oracle.identity_triplet(T, d)
        for c in perm:
            st = oracle.merge_ref(st, parts[c])
        np.testing.assert_allclose(oracle.finalize_ref(st), ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [8, 64])
def test_chunk_order_invariance_random(C):
    T, d = 6, 4
    S = 2 * C
    q, k, v = _rand((T, 1, d), C), _rand((S, 1, d), C + 1), _rand((S, 1, d), C + 2)
    ref = oracle.attention_ref(q, k, v)[:, 0]
    parts = [oracle.partial_ref(q[:, 0], k[2 * c:2 * c + 2, 0], v[2 * c:2 * c + 2, 0],
                                np.ones((T, 2), bool), 0.5) for c in range(C)]
    rng = np.random.default_rng(0)
    for _ in range(50):
        st = oracle.identity_triplet(T, d)
        for c in rng.permutation(C):
            st = oracle.merge_ref(st, parts[c])
        np.testing.assert_allclose(oracle.finalize_ref(st), ref, rtol=1e-12, atol=1e-13)


def test_dependent_trip_hand_values():
    # query tile [128, 256) against a chunk [0, 1024), block 64: active end 256 -> 4 tiles
    assert oracle.dependent_trip(0, 1024, 256, 64, causal=True) == (4, 256)
    assert oracle.dependent_trip(0, 1024, 256, 64, causal=True, prune=False) == (16, 1024)
    assert oracle.dependent_trip(0, 1024, 256, 64, causal=False) == (16, 1024)
    # ragged: tile [0, 100) -> 2 tiles of 64, the second masked at 100
    assert oracle.dependent_trip(0, 1024, 100, 64, causal=True) == (2, 100)
    # chunk entirely after the query tile: no tile
    assert oracle.dependent_trip(512, 1024, 256, 64, causal=True) == (0, 256)
    # chunk shorter than the tile end
    assert oracle.dependent_trip(0, 70, 256, 64, causal=True) == (2, 70)


def test_pruned_tile_count_closed_form():
    # square causal, n query tiles of b rows, key tiles of b: pruned visits n(n+1)/2, masked n^2
    for n in (1, 2, 8, 32):
        b = 16
        pruned = sum(oracle.dependent_trip(0, n * b, (t + 1) * b, b, True)[0] for t in range(n))
        masked = sum(oracle.dependent_trip(0, n * b, (t + 1) * b, b, True, prune=False)[0] for t in range(n))
        assert pruned == n * (n + 1) // 2 and masked == n * n


@pytest.mark.parametrize("block_k", [1, 3, 8, 64])
def test_pruning_equals_masking_bitwise(block_k):
    T, d = 40, 4
    q, k, v = _rand((T, 2, d), block_k), _rand((T, 1, d), block_k + 1), _rand((T, 1, d), block_k + 2)
    for C in (1, 4):
        a = oracle.ring_ref(q, k, v, C, causal=True, block_k=block_k, prune=True, return_triplet=True)
        b = oracle.ring_ref(q, k, v, C, causal=True, block_k=block_k, prune=False, return_triplet=True)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_attn_partial_accumulate_is_ring_step():
    T, d, C = 32, 8, 4
    q, k, v = _rand((T, 4, d), 40), _rand((T, 2, d), 41), _rand((T, 2, d), 42)
    w = T // C
    for causal in (False, True):
        st = None
        for c in (2, 0, 3, 1):
            st = oracle.attn_partial_ref(q, k[c * w:(c + 1) * w], v[c * w:(c + 1) * w], q_pos0=0,
                                         k_pos0=c * w, causal=causal, state=st)
        o = st.O / st.l[..., None]
        np.testing.assert_allclose(o, oracle.attention_ref(q, k, v, causal=causal), rtol=1e-12, atol=1e-13)
    # positions: a query block that sees none of the chunk gives the identity
    t = oracle.attn_partial_ref(q[:4], k[8:16], v[8:16], q_pos0=0, k_pos0=8, causal=True)
    assert np.all(t.m == -np.inf) and not t.l.any() and not t.O.any()


def test_ring_order_is_rotation():
    for C in (1, 2, 5, 8):
        seen = [oracle.ring_order(r, C) for r in range(C)]
        for r in range(C):
            assert sorted(seen[r]) == list(range(C)) and seen[r][0] == r
        for s in range(C):   # at every step the ranks hold all chunks once
            assert sorted(seen[r][s] for r in range(C)) == list(range(C))
        for r in range(C):   # rank r receives at step s what rank r+1 held at step s-1
            for s in range(1, C):
                assert seen[r][s] == seen[(r + 1) % C][s - 1]

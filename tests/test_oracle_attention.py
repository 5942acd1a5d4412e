"""Pins of oracle.attention_ref: brute force, a float64 library cross-check,
high-precision spot checks, closed forms and hand-derived fixtures."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests._brute import brute_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("T,S", [(1, 1), (2, 3), (3, 2), (4, 4), (7, 8), (8, 7), (8, 8)])
@pytest.mark.parametrize("d", [1, 2, 3, 4])
@pytest.mark.parametrize("heads", [(1, 1), (2, 1), (4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(T, S, d, heads, causal):
    h_q, h_kv = heads
    seed = T * 1000 + S * 100 + d * 10 + h_q + causal
    q, k, v = _rand((T, h_q, d), seed), _rand((S, h_kv, d), seed + 1), _rand((S, h_kv, d), seed + 2)
    ref = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), causal))
    got = oracle.attention_ref(q, k, v, causal=causal)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (4, 1), (8, 2)])
def test_torch_sdpa_float64(causal, heads):
    h_q, h_kv = heads
    T, d = 37, 16
    q, k, v = _rand((T, h_q, d), 5), _rand((T, h_kv, d), 6), _rand((T, h_kv, d), 7)
    g = h_q // h_kv
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, causal=causal), ref, rtol=1e-12, atol=1e-13)


def test_torch_sdpa_rectangular_mask():
    T, S, d = 5, 11, 8
    q, k, v = _rand((T, 1, d), 8), _rand((S, 1, d), 9), _rand((S, 1, d), 10)
    mask = torch.ones(T, S, dtype=torch.bool).tril()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), attn_mask=mask).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, causal=True), ref, rtol=1e-12, atol=1e-13)


def test_mpmath_50_digits():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    T, S, d = 3, 5, 4
    q, k, v = _rand((T, 1, d), 11), _rand((S, 1, d), 12), _rand((S, 1, d), 13)
    got, lse = oracle.attention_ref(q, k, v, causal=True, return_lse=True)
    for i in range(T):
        sc = [mp.mpf(1) / mp.sqrt(d) * mp.fsum(mp.mpf(q[i, 0, t]) * mp.mpf(k[j, 0, t]) for t in range(d))
              for j in range(i + 1)]
        w = [mp.e ** s for s in sc]
        den = mp.fsum(w)
        assert abs(float(mp.log(den)) - lse[i, 0]) < 1e-14
        for t in range(d):
            o = mp.fsum(w[j] * mp.mpf(v[j, 0, t]) for j in range(i + 1)) / den
            assert abs(float(o) - got[i, 0, t]) < 1e-14 * max(1.0, abs(float(o)))


def test_zero_queries_give_means():
    T, d = 9, 6
    k, v = _rand((T, 2, d), 14), _rand((T, 2, d), 15)
    q = np.zeros((T, 4, d))
    o = oracle.attention_ref(q, k, v, causal=False)
    np.testing.assert_allclose(o[:, 0], np.broadcast_to(v[:, 0].mean(0), (T, d)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[:, 3], np.broadcast_to(v[:, 1].mean(0), (T, d)), rtol=1e-13, atol=1e-14)
    oc = oracle.attention_ref(q, k, v, causal=True)
    prefix = np.cumsum(v[:, 1], axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(oc[:, 2], prefix, rtol=1e-13, atol=1e-14)


def test_zero_keys_give_means():
    T, d = 6, 3
    q, v = _rand((T, 1, d), 16), _rand((T, 1, d), 17)
    o = oracle.attention_ref(q, np.zeros((T, 1, d)), v, causal=True)
    np.testing.assert_allclose(o[:, 0], np.cumsum(v[:, 0], 0) / np.arange(1, T + 1)[:, None], rtol=1e-13)


def test_constant_values_and_single_key():
    T, S, d = 5, 7, 4
    q, k = _rand((T, 1, d), 18), _rand((S, 1, d), 19)
    c = np.array([1.5, -2.0, 0.25, 7.0])
    o = oracle.attention_ref(q, k, np.broadcast_to(c, (S, 1, d)).copy())
    np.testing.assert_allclose(o[:, 0], np.broadcast_to(c, (T, d)), rtol=1e-14)
    v = _rand((1, 1, d), 20)
    o1 = oracle.attention_ref(q, k[:1], v)
    np.testing.assert_allclose(o1[:, 0], np.broadcast_to(v[0, 0], (T, d)), rtol=1e-14)
    oc = oracle.attention_ref(q[:S], k, _rand((S, 1, d), 21), causal=True)
    assert np.array_equal(oc[0, 0], _rand((S, 1, d), 21)[0, 0])


def test_dominant_key():
    d = 8
    q = _rand((1, 1, d), 22)
    k = _rand((6, 1, d), 23)
    k[4, 0] = 200.0 * q[0, 0] / np.linalg.norm(q[0, 0])   # score >> every other
    v = _rand((6, 1, d), 24)
    o = oracle.attention_ref(q, k, v)
    np.testing.assert_allclose(o[0, 0], v[4, 0], rtol=1e-10, atol=1e-10)


def test_gqa_equals_repeated_mha():
    T, d, h_q, h_kv = 13, 8, 8, 2
    q, k, v = _rand((T, h_q, d), 25), _rand((T, h_kv, d), 26), _rand((T, h_kv, d), 27)
    g = h_q // h_kv
    for causal in (False, True):
        a = oracle.attention_ref(q, k, v, causal=causal)
        b = oracle.attention_ref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), causal=causal)
        np.testing.assert_array_equal(a, b)
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_key_permutation_invariance():
    S, d = 10, 4
    q, k, v = _rand((3, 1, d), 28), _rand((S, 1, d), 29), _rand((S, 1, d), 30)
    p = np.random.default_rng(31).permutation(S)
    np.testing.assert_allclose(oracle.attention_ref(q, k, v), oracle.attention_ref(q, k[p], v[p]), rtol=1e-13)


def test_jagged_equals_per_sequence_and_dense_batch():
    d = 4
    lens = [3, 0, 5, 1]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = offs[-1]
    q, k, v = _rand((N, 2, d), 32), _rand((N, 1, d), 33), _rand((N, 1, d), 34)
    got = oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs)
    for b in range(len(lens)):
        s0, s1 = offs[b], offs[b + 1]
        if s1 > s0:
            np.testing.assert_array_equal(got[s0:s1], oracle.attention_ref(q[s0:s1], k[s0:s1], v[s0:s1], causal=True))
    q2, k2, v2 = _rand((12, 2, d), 35), _rand((12, 2, d), 36), _rand((12, 2, d), 37)
    dense = oracle.attention_ref(q2, k2, v2, causal=True, n_seqs=3)
    jag = oracle.attention_ref(q2, k2, v2, causal=True, seq_offsets=[0, 4, 8, 12])
    np.testing.assert_array_equal(dense, jag)


def test_rows_ref_matches_full():
    lens = [5, 9, 2]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = _rand((16, 4, 8), 38), _rand((16, 2, 8), 39), _rand((16, 2, 8), 40)
    full = oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs)
    toks, heads = [0, 4, 5, 13, 14, 15], [0, 3, 1, 2, 0, 3]
    rows = oracle.attention_rows_ref(q, k, v, toks, heads, causal=True, seq_offsets=offs)
    np.testing.assert_allclose(rows, full[toks, heads], rtol=1e-13)


def test_row_blocking_does_not_change_results():
    q, k, v = _rand((50, 2, 8), 41), _rand((50, 1, 8), 42), _rand((50, 1, 8), 43)
    a = oracle.attention_ref(q, k, v, causal=True, rows_per_block=7)
    b = oracle.attention_ref(q, k, v, causal=True, rows_per_block=4096)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_hand_fixtures():
    data = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    for c in data["cases"]:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
        o, lse = oracle.attention_ref(q, k, v, causal=c["causal"], return_lse=True)
        np.testing.assert_allclose(o, np.array(c["expect_o"]), rtol=1e-14, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["expect_lse"]), rtol=1e-14, atol=1e-14, err_msg=c["name"])


def test_empty_row_is_rejected():
    with pytest.raises(ValueError):
        oracle.attention_ref(np.zeros((2, 1, 2)), np.zeros((0, 1, 2)), np.zeros((0, 1, 2)))


def _brute_rows(q, k, v, toks, heads, causal, segs, window=None):
    """Rows (tokens[n], heads[n]) by pure-Python brute force, one sequence at a
    time: segs = [(q0, q1, k0, k1)] of the packed batch."""
    out = []
    for t, h in zip(toks, heads):
        q0, q1, k0, k1 = next(s for s in segs if s[0] <= t < s[1])
        full = brute_attention(q[q0:q1].tolist(), k[k0:k1].tolist(), v[k0:k1].tolist(), causal, window)
        out.append(full[t - q0][h])
    return np.array(out)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_ref_dense_batch_brute_force(causal):
    """attention_rows_ref on a dense batch of 3 sequences (GQA 4/2): each row
    is attention over its own sequence only, with sequence-local positions."""
    n, L, d = 3, 6, 4
    q, k, v = _rand((n * L, 4, d), 44), _rand((n * L, 2, d), 45), _rand((n * L, 2, d), 46)
    toks = [0, 5, 6, 7, 11, 12, 17, 9]
    heads = [0, 3, 1, 2, 3, 0, 3, 1]
    segs = [(b * L, (b + 1) * L, b * L, (b + 1) * L) for b in range(n)]
    got = oracle.attention_rows_ref(q, k, v, toks, heads, causal=causal, n_seqs=n)
    np.testing.assert_allclose(got, _brute_rows(q, k, v, toks, heads, causal, segs), rtol=1e-12, atol=1e-13)
    full = oracle.attention_ref(q, k, v, causal=causal, n_seqs=n)
    np.testing.assert_allclose(got, full[toks, heads], rtol=1e-13, atol=1e-14)


def test_rows_ref_rectangular_noncausal_brute_force():
    """Non-causal rows of a dense batch with more keys than queries per
    sequence (T_q = 3, S_kv = 7 each): the query and key ranges differ."""
    n, Tq, Sk, d = 2, 3, 7, 5
    q, k, v = _rand((n * Tq, 2, d), 47), _rand((n * Sk, 1, d), 48), _rand((n * Sk, 1, d), 49)
    toks, heads = [0, 2, 3, 5, 4], [0, 1, 1, 0, 0]
    segs = [(b * Tq, (b + 1) * Tq, b * Sk, (b + 1) * Sk) for b in range(n)]
    got = oracle.attention_rows_ref(q, k, v, toks, heads, causal=False, n_seqs=n)
    np.testing.assert_allclose(got, _brute_rows(q, k, v, toks, heads, False, segs), rtol=1e-12, atol=1e-13)
    full = oracle.attention_ref(q, k, v, causal=False, n_seqs=n)
    np.testing.assert_allclose(got, full[toks, heads], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("window", [1, 2, 4, 9])
def test_rows_ref_window_brute_force(window):
    """Sliding-window rows (query i sees i - W < j <= i) on a dense batch of
    two sequences and on a jagged batch, against brute force."""
    d = 3
    q, k, v = _rand((16, 2, d), 50 + window), _rand((16, 1, d), 60 + window), _rand((16, 1, d), 70 + window)
    toks, heads = [0, 3, 7, 8, 12, 15], [0, 1, 1, 0, 1, 0]
    segs = [(0, 8, 0, 8), (8, 16, 8, 16)]
    got = oracle.attention_rows_ref(q, k, v, toks, heads, causal=True, n_seqs=2, window=window)
    np.testing.assert_allclose(got, _brute_rows(q, k, v, toks, heads, True, segs, window), rtol=1e-12, atol=1e-13)
    offs = [0, 5, 5, 16]
    jsegs = [(0, 5, 0, 5), (5, 16, 5, 16)]
    gotj = oracle.attention_rows_ref(q, k, v, toks, heads, causal=True, seq_offsets=offs, window=window)
    np.testing.assert_allclose(gotj, _brute_rows(q, k, v, toks, heads, True, jsegs, window), rtol=1e-12, atol=1e-13)

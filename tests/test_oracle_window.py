"""Pins of the sliding-window reading (key j admissible for query i iff
i - W < j <= i): pure-Python brute force, torch float64 SDPA with the band
mask, closed forms (W = 1 returns V itself; W >= L is plain causal), the
windowed ring and dependent-bound tile walk against the monolithic
definition (pruned == masked bit for bit), hand-derived tile ranges, and
the admissible-pair count."""
import numpy as np
import pytest
import torch

import oracle
from tests._brute import brute_attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("W", [1, 2, 3, 7])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2)])
def test_window_brute_force(T, W, heads):
    h_q, h_kv = heads
    d = 3
    q, k, v = _rand((T, h_q, d), T * 10 + W), _rand((T, h_kv, d), 1), _rand((T, h_kv, d), 2)
    ref = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), True, window=W))
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, causal=True, window=W), ref,
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("W", [1, 4, 16, 100])
def test_window_torch_sdpa_band_mask(W):
    T, d = 41, 16
    q, k, v = _rand((T, 2, d), 3), _rand((T, 2, d), 4), _rand((T, 2, d), 5)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & (i - j < W)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), attn_mask=mask).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, causal=True, window=W), ref,
                               rtol=1e-12, atol=1e-13)


def test_window_one_returns_own_value():
    q, k, v = _rand((9, 4, 8), 6), _rand((9, 2, 8), 7), _rand((9, 2, 8), 8)
    got = oracle.attention_ref(q, k, v, causal=True, window=1)
    np.testing.assert_array_equal(got, np.repeat(v, 2, axis=1))


def test_window_covering_sequence_is_causal():
    q, k, v = _rand((12, 2, 4), 9), _rand((12, 1, 4), 10), _rand((12, 1, 4), 11)
    a = oracle.attention_ref(q, k, v, causal=True)
    for W in (12, 13, 1000):
        np.testing.assert_array_equal(oracle.attention_ref(q, k, v, causal=True, window=W), a)


def test_window_zero_keys_give_band_means():
    T, W = 20, 6
    q, v = _rand((T, 1, 4), 12), _rand((T, 1, 4), 13)
    got = oracle.attention_ref(q, np.zeros((T, 1, 4)), v, causal=True, window=W)
    want = np.stack([v[max(0, i - W + 1):i + 1, 0].mean(axis=0) for i in range(T)])[:, None]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_window_jagged_is_per_sequence():
    offs = np.array([0, 7, 7, 20, 21])
    T = int(offs[-1])
    q, k, v = _rand((T, 2, 4), 14), _rand((T, 2, 4), 15), _rand((T, 2, 4), 16)
    got = oracle.attention_ref(q, k, v, causal=True, window=5, seq_offsets=offs)
    for a, b in zip(offs[:-1], offs[1:]):
        if b > a:
            np.testing.assert_allclose(got[a:b], oracle.attention_ref(q[a:b], k[a:b], v[a:b], causal=True, window=5),
                                       rtol=1e-13, atol=1e-14)


def test_window_requires_causal_and_positive():
    q = _rand((3, 1, 2), 0)
    with pytest.raises(ValueError):
        oracle.attention_ref(q, q, q, causal=False, window=2)
    with pytest.raises(ValueError):
        oracle.attention_ref(q, q, q, causal=True, window=0)


@pytest.mark.parametrize("C", [1, 2, 3, 4])
@pytest.mark.parametrize("W", [1, 5, 17, 64])
def test_window_ring_equals_monolithic(C, W):
    T = 48
    q, k, v = _rand((T, 4, 8), C * 100 + W), _rand((T, 2, 8), 1), _rand((T, 2, 8), 2)
    mono = oracle.attention_ref(q, k, v, causal=True, window=W)
    np.testing.assert_allclose(oracle.ring_ref(q, k, v, C, causal=True, window=W), mono, rtol=1e-12, atol=1e-13)
    tiled = oracle.ring_ref(q, k, v, C, causal=True, window=W, block_k=5)
    np.testing.assert_allclose(tiled, mono, rtol=1e-12, atol=1e-13)
    # the dependent lower bound and the whole-chunk skip drop only masked work
    masked = oracle.ring_ref(q, k, v, C, causal=True, window=W, block_k=5, prune=False)
    np.testing.assert_array_equal(tiled, masked)


def test_dependent_range_hand_values():
    # chunk [0, 1024), query tile [512, 576), 64-key tiles
    assert oracle.dependent_range(0, 1024, 512, 576, 64, True) == (0, 9, 0, 576)
    # window 100: first admissible key 413 -> tile 6 (keys 384..447); tiles 6..8
    assert oracle.dependent_range(0, 1024, 512, 576, 64, True, window=100) == (6, 3, 413, 576)
    # window 1: first key 512 -> tile 8 only
    assert oracle.dependent_range(0, 1024, 512, 576, 64, True, window=1) == (8, 1, 512, 576)
    # chunk [256, 512) on its own grid: first key 413 -> tile 2 (keys 384..447); end 512 -> 2 tiles
    assert oracle.dependent_range(256, 512, 512, 576, 64, True, window=100) == (2, 2, 413, 512)
    # unpruned: the whole range
    assert oracle.dependent_range(0, 1024, 512, 576, 64, True, prune=False, window=100) == (0, 16, 0, 1024)


def test_windowed_pairs():
    for L in range(0, 30):
        for W in range(1, 35):
            brute = sum(1 for i in range(L) for j in range(L) if j <= i and i - j < W)
            assert oracle.windowed_pairs(L, W) == brute
    assert oracle.prefill_pairs(8192, 8192, causal=True, window=8192) == oracle.causal_pairs(8192)
    offs = [0, 5, 5, 30]
    assert oracle.prefill_pairs(30, 30, causal=True, seq_offsets=offs, window=4) == \
        oracle.windowed_pairs(5, 4) + oracle.windowed_pairs(25, 4)

"""Planted mistakes in the oracle (CPU only): each one must make a pin fail.

This shows the pins are sensitive to the plausible slips named in the oracle's
readings: a dropped scale, the wrong GQA head mapping, a flipped rescale sign,
a normalised partial O, an off-by-one compute end, a wrong merge order in the
fan-out, and the L^2/2 pair count."""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.decode as odec
import oracle.triplet as otri
import oracle.worklist as owl
from oracle import Triplet
from tests import test_oracle_attention as A
from tests import test_oracle_triplet as TR
from tests import test_oracle_worklist_decode as WD


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "softmax_scale", lambda d: 1.0)
    _fails(A.test_torch_sdpa_float64, False, (1, 1))
    _fails(A.test_hand_fixtures)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "kv_head_of", lambda h, hq, hkv: h % hkv)
    _fails(A.test_gqa_equals_repeated_mha)
    _fails(A.test_brute_force_tiny, 4, 4, 2, (4, 2), False)


def test_flipped_rescale_sign_is_caught(monkeypatch):
    def bad_merge(a, b):
        m = np.maximum(a.m, b.m)
        shift = np.where(np.isfinite(m), m, 0.0)
        sa, sb = np.exp(shift - a.m), np.exp(b.m - shift)
        sa = np.where(np.isfinite(sa), sa, 0.0)
        return Triplet(m, a.l * sa + b.l * sb, a.O * sa[:, None] + b.O * sb[:, None])
    monkeypatch.setattr(otri, "merge_ref", bad_merge)
    _fails(TR.test_ring_equals_monolithic, 4, False, (1, 1))


def test_normalised_partial_is_caught(monkeypatch):
    good = otri.partial_ref

    def normalised(qr, kk, vv, allowed, scale):
        t = good(qr, kk, vv, allowed, scale)
        l = np.where(t.l > 0, t.l, 1.0)
        return Triplet(t.m, t.l, t.O / l[:, None])
    monkeypatch.setattr(otri, "partial_ref", normalised)
    _fails(TR.test_ring_equals_monolithic, 4, False, (1, 1))


def test_off_by_one_compute_end_is_caught(monkeypatch):
    good = owl.worklist_ref

    def bad(seq_offsets, BQ):
        return [owl.WorkItem(i.seq, i.tile, i.range_start, i.range_len, i.tile_start,
                             i.tile_extent, i.compute_end - 1) for i in good(seq_offsets, BQ)]
    monkeypatch.setattr(owl, "worklist_ref", bad)
    _fails(WD.test_worklist_hand_fixture)


def test_unordered_worklist_is_caught(monkeypatch):
    good = owl.worklist_ref
    monkeypatch.setattr(owl, "worklist_ref", lambda o, BQ: sorted(good(o, BQ), key=lambda i: (i.seq, i.tile)))
    _fails(WD.test_worklist_hand_fixture)


def test_wrong_fanout_order_is_caught(monkeypatch):
    bad = lambda r, n: [r] + [o for o in range(n) if o != r]
    monkeypatch.setattr(odec, "fanout_order", bad)
    monkeypatch.setattr(oracle, "fanout_order", bad)
    _fails(WD.test_fanout_exactly_once_and_replicated, 4)


def test_half_square_pair_count_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "causal_pairs", lambda L: L * L // 2)
    _fails(WD.test_counts_closed_forms_and_brute_force)


def test_window_off_by_one_is_caught(monkeypatch):
    from tests import test_oracle_window as WIN

    def bad_admissible(ii, jj, causal, window=None):
        ok = jj[None, :] <= ii[:, None]
        if window is not None:
            ok &= (ii[:, None] - jj[None, :]) <= window      # one key too many
        return ok
    monkeypatch.setattr(oatt, "admissible", bad_admissible)
    monkeypatch.setattr(otri, "admissible", bad_admissible)
    _fails(WIN.test_window_one_returns_own_value)
    _fails(WIN.test_window_brute_force, 5, 2, (1, 1))


def test_window_lower_bound_too_late_is_caught(monkeypatch):
    from tests import test_oracle_window as WIN
    good = otri.dependent_range

    def late(begin, kv_end, qb, qe, bk, causal, prune=True, window=None):
        first, trip, ab, ae = good(begin, kv_end, qb, qe, bk, causal, prune, window)
        if window is not None and causal and prune and trip > 1:
            return first + 1, trip - 1, ab, ae                # skips an admissible tile
        return first, trip, ab, ae
    monkeypatch.setattr(otri, "dependent_range", late)
    # a row left without keys is refused outright; others come out wrong
    for C, W in ((1, 17), (4, 64), (3, 5)):
        with pytest.raises((AssertionError, ValueError)):
            WIN.test_window_ring_equals_monolithic(C, W)


def test_decode_flops_half_count_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode_flops", lambda B, h_q, d, S: 2 * d * h_q * B * S)
    _fails(WD.test_decode_counts_brute_force)


def _rows_ref_variant(local_index: bool = True, keys_from_queries: bool = False, use_window: bool = True):
    """attention_rows_ref with one planted slip: a global instead of a
    sequence-local query index, key ranges taken from the query ranges, or
    the window dropped."""
    from oracle._util import f64, segments

    def rows(q, k, v, tokens, heads, *, causal=False, n_seqs=1, seq_offsets=None, window=None):
        T, h_q, d = q.shape
        S, h_kv, _ = k.shape
        segs = segments(T, S, n_seqs, seq_offsets)
        res = np.zeros((len(tokens), d))
        for n, (t, h) in enumerate(zip(tokens, heads)):
            q0, q1, k0, k1 = next(s for s in segs if s[0] <= t < s[1])
            if keys_from_queries:
                k0, k1 = q0, q1
            kv = oatt.kv_head_of(int(h), h_q, h_kv)
            qr = f64(q[t, h]).reshape(1, d)
            kk, vv = f64(k[k0:k1, kv]), f64(v[k0:k1, kv])
            ii = np.array([t - q0 if local_index else t])
            allowed = oatt.admissible(ii, np.arange(k1 - k0), causal, window if use_window else None)
            res[n] = oatt._attend(qr, kk, vv, allowed, oatt.softmax_scale(d))[0][0]
        return res
    return rows


def test_rows_ref_global_index_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "attention_rows_ref", _rows_ref_variant(local_index=False))
    _fails(A.test_rows_ref_dense_batch_brute_force, True)


def test_rows_ref_key_range_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "attention_rows_ref", _rows_ref_variant(keys_from_queries=True))
    with pytest.raises((AssertionError, ValueError)):
        A.test_rows_ref_rectangular_noncausal_brute_force()


def test_rows_ref_dropped_window_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "attention_rows_ref", _rows_ref_variant(use_window=False))
    _fails(A.test_rows_ref_window_brute_force, 2)

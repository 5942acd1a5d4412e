"""Partial (m, l, O) triplets, their merge, the ring fold and the dependent
causal tile bound (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "_gqa_prefill_long.py" (GQA fused-attention prefill with Ring KV): the
  step-0 partial against the local KV block (row max, exponentials shifted by
  it, their row sum, and the exponentials times V, left unnormalised), the
  online-softmax merge of each ring step into the running (m, l, O), the ring
  rotation (send west, receive from east, C - 1 steps) and the final O / l.
* "[pallas] Support dependent Tile.end bounds in Pallas": the inner KV loop
  ends at the smaller of the KV end and the enclosing query tile's end; the
  loop runs cdiv(active_end - begin, block_k) tiles and masks keys at or past
  active_end ("Unroll lowering").

Readings of what the pages leave open:
* The triplet's O is unnormalised (the prefill page's partial; the decode
  page's softmax-weighted o would be normalised twice by its own final o/l).
* An empty partial (every key masked) is the identity (-inf, 0, 0); merging two
  identities yields the identity, never exp(-inf - (-inf)).
* m is in natural-log units of the scaled score.
* Ring direction: rank r holds chunk (r + s) mod C at step s.  A query row i of
  a sequence with Lq queries belongs to rank floor(i * C / Lq).
* Jagged batches with C > 1 split each sequence into C contiguous chunks of
  ceil(L / C) keys (the last ones may be short or empty).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from ._util import f64, segments
from .attention import softmax_scale, kv_head_of, admissible


@dataclass
class Triplet:
    m: np.ndarray   # (r,)   running max of scaled scores (natural-log units)
    l: np.ndarray   # (r,)   sum of exp(s - m)
    O: np.ndarray   # (r, d) sum of exp(s - m) * V, unnormalised


def identity_triplet(rows: int, d: int) -> Triplet:
    return Triplet(np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d)))


def partial_ref(qr, kk, vv, allowed, scale) -> Triplet:
    """Triplet of rows ``qr`` (r, d) against one KV block ``kk``/``vv`` (n, d),
    restricted to ``allowed`` (r, n): m = row max of the scores, l = row sum
    of exp(score - m), O = exp(score - m) @ V.  Rows with no admissible key give
    the identity triplet."""
    qr, kk, vv = f64(qr), f64(kk), f64(vv)
    s = scale * (qr @ kk.T)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    shift = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - shift[:, None])          # masked entries: exp(-inf) = 0
    return Triplet(m, e.sum(axis=1), e @ vv)


def merge_ref(a: Triplet, b: Triplet) -> Triplet:
    """Online-softmax merge: m' = max(m_a, m_b); each side is rescaled by
    exp(m_side - m'); l and O add.  Guard: when both m are -inf the shift is 0,
    so both rescale factors are exp(-inf) = 0 and the result is the identity."""
    m = np.maximum(a.m, b.m)
    shift = np.where(np.isfinite(m), m, 0.0)
    sa = np.exp(a.m - shift)
    sb = np.exp(b.m - shift)
    return Triplet(m, a.l * sa + b.l * sb, a.O * sa[:, None] + b.O * sb[:, None])


def finalize_ref(t: Triplet) -> np.ndarray:
    """Final normalisation O / l."""
    if np.any(t.l <= 0):
        raise ValueError("finalising an empty triplet")
    return t.O / t.l[:, None]


def ring_order(r: int, C: int):
    """Chunks visited by ring rank r: (r + s) mod C for s = 0 .. C-1."""
    return [(r + s) % C for s in range(C)]


def dependent_trip(begin: int, kv_end: int, q_tile_end: int, block_k: int, causal: bool,
                   prune: bool = True):
    """(trip_count, active_end) of one KV range [begin, kv_end) for a query tile
    whose rows end (exclusive) at ``q_tile_end``.  Causal and pruned: the loop
    ends at min(kv_end, q_tile_end).  Unpruned (or non-causal): at kv_end."""
    active_end = min(kv_end, q_tile_end) if (causal and prune) else kv_end
    n = active_end - begin
    return (max(0, -(-n // block_k)), active_end)


def dependent_range(begin: int, kv_end: int, q_tile_begin: int, q_tile_end: int, block_k: int,
                    causal: bool, prune: bool = True, window=None):
    """(first_tile, trip_count, active_begin, active_end) of one KV range
    [begin, kv_end) for the query tile [q_tile_begin, q_tile_end) on a tile
    grid starting at ``begin``.  Causal and pruned: the loop ends at
    min(kv_end, q_tile_end) (the Helion page's dependent end) and, with a
    sliding window W, starts at the tile holding max(begin, q_tile_begin - W + 1)
    -- the dependent lower bound the page defers.  Unpruned: the whole range."""
    trip, active_end = dependent_trip(begin, kv_end, q_tile_end, block_k, causal, prune)
    active_begin, first = begin, 0
    if causal and prune and window is not None:
        active_begin = max(begin, q_tile_begin - window + 1)
        first = max(0, (active_begin - begin) // block_k)
        trip = max(0, trip - first)
    return first, trip, active_begin, active_end


def tiled_fold_ref(state: Triplet, qr, q_pos, kk, vv, k_pos0: int, block_k: int, causal: bool,
                   q_tile_end: int, scale: float, prune: bool = True, window=None,
                   q_tile_begin: int = 0) -> Triplet:
    """Fold one KV chunk (keys at positions k_pos0 .. k_pos0 + n - 1) into
    ``state`` tile by tile, the way the dependent-bound loop runs: tile t covers
    keys [k_pos0 + t*block_k, ... + block_k), keys at or past active_end are
    masked, and (causal) key position <= query position is required."""
    n = kk.shape[0]
    first, trip, _, active_end = dependent_range(k_pos0, k_pos0 + n, q_tile_begin, q_tile_end, block_k,
                                                 causal, prune, window)
    q_pos = np.asarray(q_pos)
    for t in range(first, first + trip):
        idx = k_pos0 + t * block_k + np.arange(block_k)
        mask_k = idx < active_end
        allowed = np.broadcast_to(mask_k[None, :], (len(q_pos), block_k))
        if causal:
            allowed = allowed & (idx[None, :] <= q_pos[:, None])
            if window is not None:
                allowed = allowed & (q_pos[:, None] - idx[None, :] < window)
        loc = np.clip(idx - k_pos0, 0, n - 1)   # masked slots never contribute
        state = merge_ref(state, partial_ref(qr, kk[loc], vv[loc], allowed, scale))
    return state


def _chunks(L: int, C: int, jagged: bool):
    if not jagged:
        if L % C:
            raise ValueError("dense ring: keys per sequence must divide by C")
        w = L // C
    else:
        w = -(-L // C) if L else 0
    return [(min(c * w, L), min((c + 1) * w, L)) for c in range(C)]


def ring_ref(q, k, v, C: int, *, causal: bool = False, n_seqs: int = 1, seq_offsets=None,
             block_k=None, prune: bool = True, return_triplet: bool = False, window=None):
    """Ring-KV prefill as the GQA prefill page runs it, one sequence at a time:
    each rank starts from the identity, visits chunks in ring order, skips a
    chunk whole when (causal) it starts at or after the rank's last query + 1
    (or, with a sliding window W, ends at or before its first query - W + 1),
    folds every other chunk (in one partial, or tile by tile with the
    dependent bounds when ``block_k`` is given), and finally divides by l."""
    q, k, v = f64(q), f64(k), f64(v)
    T, h_q, d = q.shape
    S, h_kv, _ = k.shape
    scale = softmax_scale(d)
    out = np.zeros((T, h_q, d))
    m_all, l_all = np.zeros((T, h_q)), np.zeros((T, h_q))
    for (q0, q1, k0, k1) in segments(T, S, n_seqs, seq_offsets):
        Lq, Lk = q1 - q0, k1 - k0
        if Lq == 0:
            continue
        chunks = _chunks(Lk, C, seq_offsets is not None)
        rank = (np.arange(Lq) * C) // Lq
        for h in range(h_q):
            kv = kv_head_of(h, h_q, h_kv)
            for r in range(C):
                rows = np.nonzero(rank == r)[0]
                if rows.size == 0:
                    continue
                qr = q[q0 + rows, h]
                st = identity_triplet(rows.size, d)
                last, first_row = int(rows.max()), int(rows.min())
                for c in ring_order(r, C):
                    c0, c1 = chunks[c]
                    if c1 <= c0 or (causal and c0 >= last + 1):
                        continue
                    if window is not None and prune and c1 <= first_row - window + 1:
                        continue
                    kk, vv = k[k0 + c0:k0 + c1, kv], v[k0 + c0:k0 + c1, kv]
                    if block_k is None:
                        allowed = admissible(rows, np.arange(c0, c1), causal, window)
                        st = merge_ref(st, partial_ref(qr, kk, vv, allowed, scale))
                    else:
                        st = tiled_fold_ref(st, qr, rows, kk, vv, c0, block_k, causal, last + 1,
                                            scale, prune, window, first_row)
                out[q0 + rows, h] = finalize_ref(st)
                m_all[q0 + rows, h], l_all[q0 + rows, h] = st.m, st.l
    return (out, m_all, l_all) if return_triplet else out


def attn_partial_ref(q, k, v, *, q_pos0: int = 0, k_pos0: int = 0, causal: bool = False,
                     state: Triplet | None = None):
    """Partial of all query rows against one KV chunk, as the library's
    ``attn_partial`` entry computes it: Q (T, h_q, d) at positions q_pos0.. and a
    chunk K/V (n, h_kv, d) at positions k_pos0..; causal admits key position <=
    query position.  With ``state`` (arrays shaped (T, h_q), (T, h_q),
    (T, h_q, d) packed in a Triplet) the partial is merged into it, which is one
    ring step of the GQA prefill page.  Returns a Triplet of those shapes."""
    q, k, v = f64(q), f64(k), f64(v)
    T, h_q, d = q.shape
    n, h_kv, _ = k.shape
    scale = softmax_scale(d)
    qp = q_pos0 + np.arange(T)
    kp = k_pos0 + np.arange(n)
    allowed = (kp[None, :] <= qp[:, None]) if causal else np.ones((T, n), bool)
    m, l, O = np.zeros((T, h_q)), np.zeros((T, h_q)), np.zeros((T, h_q, d))
    for h in range(h_q):
        kv = kv_head_of(h, h_q, h_kv)
        t = partial_ref(q[:, h], k[:, kv], v[:, kv], allowed, scale)
        if state is not None:
            t = merge_ref(Triplet(f64(state.m)[:, h], f64(state.l)[:, h], f64(state.O)[:, h]), t)
        m[:, h], l[:, h], O[:, h] = t.m, t.l, t.O
    return Triplet(m, l, O)

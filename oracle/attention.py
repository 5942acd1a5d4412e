"""Monolithic scaled-dot-product attention, the plain definition (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (for every sequence, query head h and query row i):

    s_ij = scale * <Q[i, h, :], K[j, kv(h), :]>          scale = 1 / sqrt(d)
    O[i, h, :] = sum_{j in A(i)} exp(s_ij - M_i) V[j, kv(h), :] / sum_{j in A(i)} exp(s_ij - M_i)
    M_i = max_{j in A(i)} s_ij,    LSE_i = M_i + ln sum_{j in A(i)} exp(s_ij - M_i)

Readings of what the pages leave open:

* Scale.  The GQA prefill page lists the softmax scale as omitted (a deviation
  of the simulator kernel); the build applies 1/sqrt(d) everywhere.
* K^T.  That page loads K through a byte-conserving reshape that is only right
  for zero or symmetric inputs; the reading here is a true transpose, s = Q K^T.
* GQA.  The mesh decode page groups consecutive query heads per KV head
  (8 query heads per KV group at its headline scale); query head h reads KV
  head floor(h / g), g = h_q / h_kv.
* Causal.  The Helion page bounds the KV loop by the query tile's end; the
  element-level rule used here is key j admissible for query i iff j <= i,
  with query and key indices local to the sequence (top-left alignment).
* Sliding window.  The Helion page ("Scalar minimum") leaves dependent lower
  bounds to a later sliding-window feature without defining it; the reading
  here is the causal window of W keys ending at the query: key j admissible
  for query i iff i - W < j <= i (W >= 1; W = 1 is the query's own key, and
  W >= the sequence length is plain causal attention).
"""
from __future__ import annotations

import math

import numpy as np

from ._util import f64, segments


def softmax_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def kv_head_of(h: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head h: contiguous groups of g = h_q / h_kv."""
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    return h // (h_q // h_kv)


def _attend(qr: np.ndarray, kk: np.ndarray, vv: np.ndarray, allowed: np.ndarray, scale: float):
    """Softmax attention of rows ``qr`` (r, d) over keys ``kk`` / values ``vv``
    (n, d) restricted to the boolean mask ``allowed`` (r, n)."""
    s = scale * (qr @ kk.T)
    s = np.where(allowed, s, -np.inf)
    M = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(M)):
        raise ValueError("a query row has no admissible key; attention is undefined there")
    e = np.exp(s - M)
    den = e.sum(axis=1, keepdims=True)
    return (e @ vv) / den, M[:, 0] + np.log(den[:, 0])


def admissible(ii: np.ndarray, jj: np.ndarray, causal: bool, window=None) -> np.ndarray:
    """Boolean (len(ii), len(jj)): key jj admissible for query ii (sequence-
    local indices) under the causal rule and, if given, the sliding window."""
    if window is not None:
        if not causal:
            raise ValueError("a sliding window is defined for causal attention only")
        if window < 1:
            raise ValueError("window must be >= 1")
    if not causal:
        return np.ones((len(ii), len(jj)), bool)
    ok = jj[None, :] <= ii[:, None]
    if window is not None:
        ok &= (ii[:, None] - jj[None, :]) < window
    return ok


def attention_ref(q, k, v, *, causal: bool = False, n_seqs: int = 1, seq_offsets=None,
                  return_lse: bool = False, rows_per_block: int = 4096, window=None):
    """O (tokens, h_q, d) float64 for Q (tokens, h_q, d), K/V (tokens, h_kv, d).

    Dense batch when ``seq_offsets`` is None (``n_seqs`` equal sequences),
    otherwise a jagged self-attention batch packed by the int prefix offsets.
    Rows are evaluated ``rows_per_block`` at a time purely to bound memory:
    each output row depends only on its own definition above."""
    q, k, v = f64(q), f64(k), f64(v)
    T, h_q, d = q.shape
    S, h_kv, _ = k.shape
    scale = softmax_scale(d)
    out = np.zeros((T, h_q, d))
    lse = np.zeros((T, h_q))
    for (q0, q1, k0, k1) in segments(T, S, n_seqs, seq_offsets):
        jj = np.arange(k1 - k0)
        for h in range(h_q):
            kv = kv_head_of(h, h_q, h_kv)
            kk, vv = k[k0:k1, kv], v[k0:k1, kv]
            for r0 in range(q0, q1, rows_per_block):
                r1 = min(q1, r0 + rows_per_block)
                ii = np.arange(r0 - q0, r1 - q0)
                allowed = admissible(ii, jj, causal, window)
                o, l = _attend(q[r0:r1, h], kk, vv, allowed, scale)
                out[r0:r1, h] = o
                lse[r0:r1, h] = l
    return (out, lse) if return_lse else out


def attention_rows_ref(q, k, v, tokens, heads, *, causal: bool = False, n_seqs: int = 1,
                       seq_offsets=None, window=None):
    """Selected output rows O[tokens[n], heads[n], :] (float64, (n, d)), each
    evaluated from the definition on its own (for spot checks at full size)."""
    T, h_q, d = q.shape
    S, h_kv, _ = k.shape
    segs = segments(T, S, n_seqs, seq_offsets)
    starts = np.array([s[0] for s in segs])
    scale = softmax_scale(d)
    res = np.zeros((len(tokens), d))
    for n, (t, h) in enumerate(zip(tokens, heads)):
        b = int(np.searchsorted(starts, t, side="right") - 1)
        while segs[b][1] <= t:  # skip empty sequences sharing the same start
            b += 1
        q0, q1, k0, k1 = segs[b]
        kv = kv_head_of(int(h), h_q, h_kv)
        qr = f64(q[t, h]).reshape(1, d)
        kk, vv = f64(k[k0:k1, kv]), f64(v[k0:k1, kv])
        jj = np.arange(k1 - k0)
        allowed = admissible(np.array([t - q0]), jj, causal, window)
        res[n] = _attend(qr, kk, vv, allowed, scale)[0][0]
    return res

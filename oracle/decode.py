"""Split-KV decode: per-chunk partial triplets, their merge, and the
bidirectional triplet fan-out (fp64, CPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "_attention_mesh_mlo.py" (mesh-native bidirectional mlo decode).
Every rank holds the (small) query and a sequence slice of K/V that stays in
place; it computes one local partial (scores, their max m, ell = sum of
exp(scores - m), o), then runs n - 1 fan-out steps: a rank with an east
neighbour sends east, one with a west neighbour sends west, it merges what
arrives from the west (origin rank - step) and then from the east (origin
rank + step) into its running state with the same max-rescale rule as the
prefill page, and forwards the triplet it received (not its merged state).
The final answer o / ell ends up on every rank.

Readings:
* The page forms o from the normalised softmax but still divides by ell at
  the end; o is read as unnormalised exp(scores - m) @ V (see triplet.py).
* The page views K as one (h_q * d, S) block, which contracts across heads
  and does not conserve bytes when h_q != h_kv; the reading is per-head
  attention, query head h using KV head floor(h / g).
* The KV slice of a rank is a chunk of ceil(S / n) consecutive keys (the last
  chunks may be short or empty; an empty chunk yields the identity).
* The "merge tree" is a balanced pairwise tree; any order gives the same
  exact result, which the tests check.
"""
from __future__ import annotations

from collections import deque

import numpy as np

from ._util import f64
from .attention import softmax_scale, kv_head_of
from .triplet import Triplet, identity_triplet, partial_ref, merge_ref, finalize_ref


def _chunk_bounds(S: int, n_chunks: int):
    w = -(-S // n_chunks)
    return [(min(c * w, S), min((c + 1) * w, S)) for c in range(n_chunks)]


def decode_partials_ref(q, k, v, n_chunks: int):
    """Local partial of every (sequence b, query head h, chunk c).
    q (B, h_q, d); k, v (B, S, h_kv, d).  Returns m, l (B, h_q, C) and
    O (B, h_q, C, d), O unnormalised."""
    q, k, v = f64(q), f64(k), f64(v)
    B, h_q, d = q.shape
    _, S, h_kv, _ = k.shape
    scale = softmax_scale(d)
    m = np.zeros((B, h_q, n_chunks)); l = np.zeros((B, h_q, n_chunks))
    O = np.zeros((B, h_q, n_chunks, d))
    for b in range(B):
        for c, (s0, s1) in enumerate(_chunk_bounds(S, n_chunks)):
            for h in range(h_q):
                kv = kv_head_of(h, h_q, h_kv)
                if s1 > s0:
                    t = partial_ref(q[b, h][None], k[b, s0:s1, kv], v[b, s0:s1, kv],
                                    np.ones((1, s1 - s0), bool), scale)
                else:
                    t = identity_triplet(1, d)
                m[b, h, c], l[b, h, c], O[b, h, c] = t.m[0], t.l[0], t.O[0]
    return m, l, O


def _triplets_of(m, l, O):
    return [Triplet(np.atleast_1d(m[c]), np.atleast_1d(l[c]), np.atleast_2d(O[c]))
            for c in range(len(m))]


def tree_merge_ref(ts):
    """Balanced pairwise merge: neighbours pair up level by level, an odd one
    out is carried to the next level."""
    ts = list(ts)
    while len(ts) > 1:
        nxt = [merge_ref(ts[i], ts[i + 1]) for i in range(0, len(ts) - 1, 2)]
        if len(ts) % 2:
            nxt.append(ts[-1])
        ts = nxt
    return ts[0]


def fanout_order(rank: int, n: int):
    """Origins in the order rank ``rank`` merges them in the fan-out: its own,
    then per step s the one from the west (rank - s) and the one from the east
    (rank + s), when those ranks exist."""
    order = [rank]
    for s in range(1, n):
        if rank - s >= 0:
            order.append(rank - s)
        if rank + s < n:
            order.append(rank + s)
    return order


def chain_merge_ref(ts, rank: int):
    order = fanout_order(rank, len(ts))
    st = ts[order[0]]
    for c in order[1:]:
        st = merge_ref(st, ts[c])
    return st


def splitkv_decode_ref(q, k, v, n_chunks: int, order: str = "tree", rank: int = 0):
    """O (B, h_q, d): per-chunk partials merged in ``order`` ("tree",
    "linear", or "chain" = the fan-out order seen by ``rank``), then o / ell."""
    m, l, O = decode_partials_ref(q, k, v, n_chunks)
    B, h_q, C, d = O.shape
    out = np.zeros((B, h_q, d))
    for b in range(B):
        for h in range(h_q):
            ts = _triplets_of(m[b, h], l[b, h], O[b, h])
            if order == "tree":
                st = tree_merge_ref(ts)
            elif order == "linear":
                st = ts[0]
                for t in ts[1:]:
                    st = merge_ref(st, t)
            elif order == "chain":
                st = chain_merge_ref(ts, rank)
            else:
                raise ValueError(order)
            out[b, h] = finalize_ref(st)[0]
    return out


def fanout_simulate(ts, merge=merge_ref):
    """Message-level simulation of the bidirectional fan-out over an open chain
    of n ranks.  Links are FIFO queues; in each step every rank first sends,
    then receives.  Returns (final triplet per rank, per-rank log of
    (step, origin) in merge order)."""
    n = len(ts)
    east = {r: deque() for r in range(n)}   # messages travelling r -> r+1
    west = {r: deque() for r in range(n)}   # messages travelling r -> r-1
    state = list(ts)
    log = [[] for _ in range(n)]
    send_e = [(r, ts[r]) for r in range(n)]
    send_w = [(r, ts[r]) for r in range(n)]
    for step in range(1, n):
        for r in range(n):
            if r < n - 1 and send_e[r] is not None:
                east[r].append(send_e[r])
            if r > 0 and send_w[r] is not None:
                west[r].append(send_w[r])
        got_w, got_e = [None] * n, [None] * n
        for r in range(n):
            if r > 0 and r - step >= 0:
                got_w[r] = east[r - 1].popleft()
                state[r] = merge(state[r], got_w[r][1])
                log[r].append((step, got_w[r][0]))
            if r < n - 1 and r + step < n:
                got_e[r] = west[r + 1].popleft()
                state[r] = merge(state[r], got_e[r][1])
                log[r].append((step, got_e[r][0]))
        send_e, send_w = got_w, got_e
    leftover = sum(len(q) for q in east.values()) + sum(len(q) for q in west.values())
    if leftover:
        raise AssertionError(f"{leftover} triplets sent but never received")
    return state, log

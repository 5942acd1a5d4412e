"""Work and traffic counts that define the reported rates (exact ints).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Helion page reports causal "useful" TF/s.  Reading: useful FLOPs count
2d for the score and 2d for the value product of every admissible (query,
key) pair, per query head, i.e. 4 * d * h_q * pairs; a causal sequence of
length L has L (L + 1) / 2 admissible pairs (key position <= query position).
Decode traffic counts each algorithmically necessary byte once: K and V read
once per KV head, the query read and the output written once.
"""
from __future__ import annotations

import numpy as np


def causal_pairs(L: int) -> int:
    return L * (L + 1) // 2


def windowed_pairs(L: int, W: int) -> int:
    """Admissible pairs of a causal sliding window of W keys over L tokens:
    query i sees min(i + 1, W) keys."""
    if W >= L:
        return causal_pairs(L)
    return causal_pairs(W) + (L - W) * W


def prefill_pairs(T_q: int, S_kv: int, *, causal: bool, n_seqs: int = 1, seq_offsets=None,
                  window=None) -> int:
    if window is not None:
        if not causal:
            raise ValueError("a sliding window is defined for causal attention only")
        Ls = (np.diff(np.asarray(seq_offsets, dtype=np.int64)) if seq_offsets is not None
              else [T_q // n_seqs] * n_seqs)
        return int(sum(windowed_pairs(int(L), window) for L in Ls))
    if seq_offsets is not None:
        Ls = np.diff(np.asarray(seq_offsets, dtype=np.int64))
        if causal:
            return int(sum(causal_pairs(int(L)) for L in Ls))
        return int(sum(int(L) * int(L) for L in Ls))
    tq, sk = T_q // n_seqs, S_kv // n_seqs
    if causal:
        if tq != sk:
            raise ValueError("causal pairs are defined for square sequences")
        return n_seqs * causal_pairs(tq)
    return n_seqs * tq * sk


def useful_flops_prefill(h_q: int, d: int, pairs: int) -> int:
    return 4 * d * h_q * pairs


def decode_bytes(B: int, h_q: int, h_kv: int, d: int, S: int, elem_bytes: int = 2) -> int:
    kv = 2 * B * S * h_kv * d * elem_bytes
    qo = 2 * B * h_q * d * elem_bytes
    return kv + qo


def decode_flops(B: int, h_q: int, d: int, S: int) -> int:
    return 4 * d * h_q * B * S

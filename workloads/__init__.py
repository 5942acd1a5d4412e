"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This module holds shapes, seeds and random-number draws only. It contains none
of the attention arithmetic, so that neither side can borrow the other's math
through it.

Workloads (shapes follow the pages' problems; all values are i.i.d. N(0, 1)):

* ``ring_tiny``   -- one head, 128 queries against 512 keys split into 4 ring
  chunks, d = 64, fp32, non-causal (the ring step of the GQA prefill kernel
  page, "Steps 1..C-1" block, at a size a CPU checks in milliseconds).
* ``gqa_ring``    -- GQA ring prefill, 32 query heads over 8 KV heads, d = 128,
  8192 tokens in 8 chunks, bf16, causal.
* ``dense_causal``-- the dense causal flash table of the Helion Pallas page
  ("Results: Dense causal flash"): 8 sequences x 4096 tokens, 32 heads, d = 256, bf16.
* ``jagged``      -- the jagged causal table of the same page ("Results: jagged
  causal self-attn"): 1152 sequences, 4 heads, d = 128, bf16.  The page does
  not give its length distribution; lengths are drawn uniformly from
  [64, 2048] with numpy's PCG64 seeded 0.
* ``gqa_swa``     -- the ``gqa_ring`` shape with a causal sliding window of 2048
  keys (the dependent lower bound the Helion page defers to sliding-window
  support), seed 6.
* ``decode``      -- split-KV GQA decode in the shape of the mesh decode page's
  headline scale: 8 sequences, 64 query heads over 8 KV heads, d = 128,
  131072 cached keys per sequence in 64 chunks, bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "jagged_lengths", "seq_offsets_from_lengths",
           "randn", "make_prefill_inputs", "make_decode_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    dtype: str                # "f32" or "bf16"
    h_q: int
    h_kv: int
    d: int
    seed: int
    # prefill
    n_seqs: int = 1
    T_q: int = 0              # queries per sequence (dense batch)
    S_kv: int = 0             # keys per sequence (dense batch)
    C: int = 1
    causal: bool = False
    jagged: bool = False
    window: Optional[int] = None   # causal sliding window (keys), None = none
    # decode
    B: int = 0
    S_cache: int = 0
    n_chunks: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    "ring_tiny": Workload("ring_tiny", "prefill", "f32", h_q=1, h_kv=1, d=64, seed=1,
                          T_q=128, S_kv=512, C=4, causal=False),
    "gqa_ring": Workload("gqa_ring", "prefill", "bf16", h_q=32, h_kv=8, d=128, seed=2,
                         T_q=8192, S_kv=8192, C=8, causal=True),
    "dense_causal": Workload("dense_causal", "prefill", "bf16", h_q=32, h_kv=32, d=256, seed=3,
                             n_seqs=8, T_q=4096, S_kv=4096, C=1, causal=True),
    "jagged": Workload("jagged", "prefill", "bf16", h_q=4, h_kv=4, d=128, seed=4,
                       n_seqs=1152, C=1, causal=True, jagged=True),
    "gqa_swa": Workload("gqa_swa", "prefill", "bf16", h_q=32, h_kv=8, d=128, seed=6,
                        T_q=8192, S_kv=8192, C=8, causal=True, window=2048),
    "decode": Workload("decode", "decode", "bf16", h_q=64, h_kv=8, d=128, seed=5,
                       B=8, S_cache=131072, n_chunks=64),
}


def jagged_lengths(n_seqs: int = 1152, lo: int = 64, hi: int = 2048, seed: int = 0) -> np.ndarray:
    """Sequence lengths drawn uniformly from the integers [lo, hi] (inclusive)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=n_seqs).astype(np.int64)


def seq_offsets_from_lengths(lengths) -> np.ndarray:
    """Prefix offsets (n+1 int32 entries, first 0) of packed sequences."""
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    if out[-1] >= 2**31:
        raise ValueError("packed token count exceeds int32")
    return out.astype(np.int32)


def _torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def randn(shapes, seed: int, dtype: str = "f32", device="cpu"):
    """Draw one N(0,1) fp32 tensor per shape, in order, from one seeded generator,
    then round to ``dtype`` (bf16 rounding is round-to-nearest-even).

    The same (shapes, seed, device) always gives bit-identical tensors.  Host
    and device generators are different streams, so a test that compares two
    implementations hands both the very same tensors."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    out = []
    for shp in shapes:
        x = torch.randn(tuple(int(s) for s in shp), generator=g, dtype=torch.float32, device=dev)
        out.append(x.to(_torch_dtype(dtype)) if dtype != "f32" else x)
    return out


def make_prefill_inputs(w: Workload, device="cpu", lengths: Optional[np.ndarray] = None):
    """Q (tokens, h_q, d), K and V (tokens, h_kv, d) and, for jagged workloads,
    int32 seq_offsets.  Returns (q, k, v, seq_offsets_or_None)."""
    if w.jagged:
        if lengths is None:
            lengths = jagged_lengths(w.n_seqs)
        offs = seq_offsets_from_lengths(lengths)
        tq = tk = int(offs[-1])
    else:
        offs = None
        tq, tk = w.n_seqs * w.T_q, w.n_seqs * w.S_kv
    q, k, v = randn([(tq, w.h_q, w.d), (tk, w.h_kv, w.d), (tk, w.h_kv, w.d)],
                    w.seed, w.dtype, device)
    return q, k, v, offs


def make_decode_inputs(w: Workload, device="cpu"):
    """q (B, h_q, d) -- one query token per sequence -- and the KV cache
    K, V (B, S_cache, h_kv, d)."""
    return tuple(randn([(w.B, w.h_q, w.d), (w.B, w.S_cache, w.h_kv, w.d),
                        (w.B, w.S_cache, w.h_kv, w.d)], w.seed, w.dtype, device))

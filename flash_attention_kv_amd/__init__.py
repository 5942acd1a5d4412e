"""flash_attention_kv_amd -- MI355X (gfx950) blockwise attention with
(m, l, O) triplet merging: ring-KV prefill (GQA, causal with dependent-end
pruning, jagged batches) and split-KV decode.

The computation lives in hand-written HIP kernels behind the C ABI of
``include/fakv.h`` (libfakv.so, built in-tree by
``python -m flash_attention_kv_amd.build``).  This package is the thin Python
binding: PyTorch supplies device memory and the HIP stream only.
"""
from ._binding import (F32, BF16, FakvError, LIB_PATH, SIGNATURES, lib, ring_attn_fwd,
                       attn_partial, lse_merge, splitkv_decode, jagged_worklist, query_tile_rows,
                       ring_attn_workspace_bytes, splitkv_decode_workspace_bytes,
                       splitkv_decode_noalloc, DECODE_SCRATCH_BYTES)

__all__ = ["F32", "BF16", "FakvError", "LIB_PATH", "SIGNATURES", "lib", "ring_attn_fwd",
           "attn_partial", "lse_merge", "splitkv_decode", "jagged_worklist", "query_tile_rows",
           "ring_attn_workspace_bytes", "splitkv_decode_workspace_bytes",
           "splitkv_decode_noalloc", "DECODE_SCRATCH_BYTES"]

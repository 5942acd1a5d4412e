"""CPU oracle for blockwise attention with (m, l, O) triplet merging.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
fp64 NumPy statement of what the GPU library computes.  Only the test suite,
the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls it, and it shares no
code with the GPU library: the only module both sides use is ``workloads``,
which draws seeded random inputs and holds none of the method's arithmetic.

Sources (web pages, cited by title and section):

* "[pallas] Support dependent Tile.end bounds in Pallas" (Helion pull request):
  the dependent causal end of the inner KV loop ("Bound recognition",
  "Unroll lowering"), flattened worklists ("Flattened worklists") and the
  result tables.
* "_gqa_prefill_long.py" (kernbench2, GQA fused-attention prefill with Ring KV):
  the per-block partial (m, l, O), the online-softmax merge, the ring rotation
  and the final O / l.
* "_attention_mesh_mlo.py" (kernbench2, mesh-native bidirectional mlo decode):
  the one-shot local partial of sequence-sharded decode and the bidirectional
  fan-out of (m, l, o) triplets.

Every function either writes out a closed-form definition or follows the
pages' algorithm step by step; library primitives (matmul, exp, max) serve as
steps, with no blocking or fusion the definition does not state.  Readings of
points the pages leave open are listed in each function's docstring.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (brute force, closed forms, a float64 library
cross-check, high-precision spot checks, hand-derived fixtures and the pages'
invariants).  No function is "parity unpinned".
"""
from .attention import attention_ref, attention_rows_ref, softmax_scale, kv_head_of, admissible
from .triplet import (Triplet, identity_triplet, partial_ref, merge_ref, finalize_ref,
                      ring_order, ring_ref, dependent_trip, dependent_range, tiled_fold_ref,
                      attn_partial_ref)
from .worklist import WorkItem, worklist_ref, worklist_array_ref
from .decode import (decode_partials_ref, splitkv_decode_ref, tree_merge_ref, chain_merge_ref,
                     fanout_order, fanout_simulate)
from .counts import (causal_pairs, windowed_pairs, prefill_pairs, useful_flops_prefill, decode_bytes,
                     decode_flops)

__all__ = [
    "attention_ref", "attention_rows_ref", "softmax_scale", "kv_head_of",
    "Triplet", "identity_triplet", "partial_ref", "merge_ref", "finalize_ref",
    "ring_order", "ring_ref", "dependent_trip", "tiled_fold_ref", "attn_partial_ref",
    "WorkItem", "worklist_ref", "worklist_array_ref",
    "decode_partials_ref", "splitkv_decode_ref", "tree_merge_ref", "chain_merge_ref",
    "fanout_order", "fanout_simulate",
    "causal_pairs", "prefill_pairs", "useful_flops_prefill", "decode_bytes", "decode_flops",
]

"""Grouping two query tiles per workgroup on jagged batches.

A jagged bf16 batch runs workgroups of twice the query rows of a dense one,
so two query tiles share each K/V tile brought into LDS ("[pallas] Support
dependent Tile.end bounds in Pallas", "Flattened worklists": the grouping-2
work bodies that share a resident cache).  Each wave still owns its 32 query
rows and visits exactly the tiles those rows admit, in the same ring order,
so where both use key tiles of the same width a jagged batch of equal-length
sequences must reproduce the dense batch of the same sequences bit for bit
(chunk width a multiple of both tile heights), and both must match the
oracle.  Dense d = 128 batches without a window walk 128-key tiles (the
jagged ones 64-key tiles): the online softmax then folds the keys in other
groups, so there the two are each held to the oracle instead."""
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("d,heads,C,window", [
    (128, (8, 2), 1, None),
    (128, (4, 4), 4, None),
    (64, (6, 3), 2, None),
    (256, (4, 1), 4, None),
    (128, (8, 2), 4, 300),
    (256, (2, 2), 1, 77),
])
def test_jagged_equal_lengths_match_dense(d, heads, C, window):
    h_q, h_kv = heads
    n, L = 3, 1024
    q, k, v = randn([(n * L, h_q, d), (n * L, h_kv, d), (n * L, h_kv, d)], 31 + d + C, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    offs = torch.from_numpy(seq_offsets_from_lengths([L] * n)).to(DEV)
    dense = F.ring_attn_fwd(qd, kd, vd, C=C, causal=True, n_seqs=n, window=window)
    jag = F.ring_attn_fwd(qd, kd, vd, C=C, causal=True, seq_offsets=offs, window=window)
    torch.cuda.synchronize()
    assert F.query_tile_rows(h_q, h_kv, d) > 0
    same_tiles = not (d == 128 and window is None)
    if same_tiles:
        assert torch.equal(dense, jag), f"d={d} heads={heads} C={C} W={window}"
    # one sequence against the oracle (the others are the same computation)
    ref = oracle.ring_ref(q[:L], k[:L], v[:L], C, causal=True, window=window)
    check(host(jag[:L]), ref, "bf16", f"grouped jagged d={d} {heads} C={C} W={window}")
    if not same_tiles:
        check(host(dense[:L]), ref, "bf16", f"dense d={d} {heads} C={C} W={window}")


def test_grouped_tile_straddles_sequence_end():
    """Lengths one past, one short of and inside a grouped tile: the second
    half of a workgroup may hold no rows at all, or a ragged few."""
    h_q, h_kv, d = 8, 2, 128
    bq = F.query_tile_rows(h_q, h_kv, d)
    lens = [bq + 1, bq - 1, bq // 2, bq // 2 + 1, 1, 2 * bq + 33]
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = randn([(N, h_q, d), (N, h_kv, d), (N, h_kv, d)], 5, "bf16")
    o = F.ring_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True,
                        seq_offsets=torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.ring_ref(q, k, v, 1, causal=True, seq_offsets=offs)
    check(host(o), ref, "bf16", f"grouped tile edges {lens}")

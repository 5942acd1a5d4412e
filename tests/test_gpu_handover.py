"""Item hand-over in persistent jagged workgroups.

A jagged bf16 batch is drained by persistent workgroups that run many work
items (query tiles of the "[pallas] Support dependent Tile.end bounds in
Pallas" page's flattened worklist) one after another.  With one ring chunk,
causal and pruned, a wave whose rows need no more key tiles of an item writes
its output before the item ends and copies its Q rows of the next item into
LDS.  Which items a workgroup runs, and in what order, depends on the atomic
queue counters, so the result must not depend on it: a batch must equal,
bit for bit, the same sequences run as two separate batches (other item
chains, other hand-overs), and match the oracle.  The batches here are large
enough that every workgroup runs a chain of items."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _lengths(seed: int, n: int = 700):
    """Mixed lengths: uniform ones plus the edges of 32-row wave slices,
    64-key tiles and 256-row items (and empty sequences)."""
    r = np.random.default_rng(seed)
    lens = r.integers(1, 900, size=n)
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 768, 1024]
    lens[r.choice(n, size=len(edges), replace=False)] = edges
    return lens


def _run(q, k, v, lens, window):
    offs = torch.from_numpy(seq_offsets_from_lengths(lens)).to(DEV)
    return F.ring_attn_fwd(q, k, v, C=1, causal=True, seq_offsets=offs, window=window)


@pytest.mark.parametrize("d,heads,window", [
    (128, (4, 4), None),
    (128, (8, 2), None),
    (64, (4, 4), None),
    (128, (4, 4), 300),
    (128, (32, 8), None),
])
def test_batch_equals_split_batches_and_oracle(d, heads, window):
    h_q, h_kv = heads
    lens = _lengths(11 + d + h_q, 700 if h_q <= 8 else 200)   # >= ~12 items per workgroup either way
    offs = seq_offsets_from_lengths(lens)
    N = int(offs[-1])
    q, k, v = randn([(N, h_q, d), (N, h_kv, d), (N, h_kv, d)], 3 + h_q, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    whole = _run(qd, kd, vd, lens, window)
    cut = len(lens) // 2
    t = int(offs[cut])
    first = _run(qd[:t], kd[:t], vd[:t], lens[:cut], window)
    second = _run(qd[t:], kd[t:], vd[t:], lens[cut:], window)
    again = _run(qd, kd, vd, lens, window)
    torch.cuda.synchronize()
    tag = f"d={d} heads={heads} W={window}"
    assert torch.equal(whole, again), f"two runs differ: {tag}"
    assert torch.equal(whole[:t], first), f"first half differs from its own batch: {tag}"
    assert torch.equal(whole[t:], second), f"second half differs from its own batch: {tag}"
    # the oracle on the longest sequence and the tile-edge lengths
    pick = [int(np.argmax(lens))] + [int(np.where(lens == e)[0][0]) for e in (33, 255, 257, 513)]
    for i in pick:
        a, b = int(offs[i]), int(offs[i + 1])
        ref = oracle.attention_ref(q[a:b], k[a:b], v[a:b], causal=True, window=window)
        check(host(whole[a:b]), ref, "bf16", f"{tag} sequence {i} (L={b - a})")

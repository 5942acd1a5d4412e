"""GPU tests of the jagged pre-pass of ring_attn_fwd (bf16).  Batches of at
most 2048 sequences and 12288 worklist slots build the worklist and the
per-XCD queues in one fused launch, larger ones in two (worklist, then
schedule).  Either way the records in the workspace must equal the ones
fakv_jagged_worklist builds, bit for bit ("[pallas] Support dependent
Tile.end bounds in Pallas", "Flattened worklists": the item list itself),
every (record, head group) entry must sit in exactly one queue once, and the
output must match the oracle.

The workspace layout read here is the library's own: n_items at byte 0, the
8 queue lengths at byte 64, the records from byte 256, then (each padded to
256 bytes) the (sequence, tile) map, the tile prefix sums, the ranking and
the 8 queues of capacity * head groups entries each."""
import numpy as np
import pytest
import torch

import flash_attention_kv_amd as F
import oracle
from tests._gpu import check, host
from workloads import randn, seq_offsets_from_lengths

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _a256(x: int) -> int:
    return (x + 255) & ~255


def _lengths(kind: str) -> np.ndarray:
    rng = np.random.default_rng({"long": 5, "at_limit": 6, "beyond": 7, "big_items": 8}[kind])
    if kind == "long":          # few sequences, several longer than 2048 tokens, some empty
        lens = rng.integers(0, 2600, size=24)
        lens[::7] = 0
    elif kind == "at_limit":    # exactly the fused kernel's sequence limit
        lens = rng.integers(0, 200, size=2048)
    elif kind == "beyond":      # more sequences than the fused kernel holds
        lens = rng.integers(0, 60, size=2600)
        lens[::13] = 0
    else:                       # few sequences, but more worklist slots than the fused kernel holds
        lens = np.full(48, 65536, dtype=np.int64)
    return lens.astype(np.int64)


@pytest.mark.parametrize("kind,heads", [("long", (4, 4)), ("long", (8, 2)), ("at_limit", (4, 4)),
                                        ("beyond", (4, 4)), ("beyond", (8, 2))])
def test_prepass_records_queues_and_output(kind, heads):
    h_q, h_kv = heads
    d = 128
    lens = _lengths(kind)
    offs = seq_offsets_from_lengths(lens)
    N, n = int(offs[-1]), len(lens)
    q, k, v = randn([(N, h_q, d), (N, h_kv, d), (N, h_kv, d)], 40 + n, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    offs_d = torch.from_numpy(offs).to(DEV)
    need = F.ring_attn_workspace_bytes(N, N, h_q, h_kv, d, 1, True, n, True, F.BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o = F.ring_attn_fwd(qd, kd, vd, causal=True, seq_offsets=offs_d, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)

    BQ = F.query_tile_rows(h_q, h_kv, d)
    n_hg = h_q // (256 // BQ)                  # 8 waves of 32 rows: 256 / BQ query heads per workgroup
    cap = N // BQ + n
    n_items = int(w[0])
    recs = w[64:64 + 8 * n_items].reshape(n_items, 8)
    ref_items, ref_n = F.jagged_worklist(offs_d, N, BQ)
    torch.cuda.synchronize()
    assert n_items == int(ref_n.item()) == int(sum((L + BQ - 1) // BQ for L in lens))
    assert np.array_equal(recs, ref_items[:n_items].cpu().numpy()), kind

    o_sched = (256 + _a256(cap * 32) + _a256(cap * 4) + _a256((n + 1) * 4) + _a256(n * 4)) // 4
    stride = cap * n_hg
    qlen = w[16:24]
    entries = np.concatenate([w[o_sched + x * stride:o_sched + x * stride + int(qlen[x])] for x in range(8)])
    assert np.array_equal(np.sort(entries), np.arange(n_items * n_hg)), kind

    check(host(o), oracle.attention_ref(q, k, v, causal=True, seq_offsets=offs), "bf16", f"pre-pass {kind} {heads}")


def test_prepass_beyond_item_limit_matches_worklist():
    """More worklist slots than the fused kernel holds (few, long sequences):
    the two-kernel path, records only (the output of such long sequences is
    covered by the full-size tests)."""
    lens = _lengths("big_items")
    offs = seq_offsets_from_lengths(lens)
    N, n = int(offs[-1]), len(lens)
    h_q = h_kv = 1
    d = 64
    q, k, v = (torch.zeros((N, h, d), dtype=torch.bfloat16, device=DEV) for h in (h_q, h_kv, h_kv))
    offs_d = torch.from_numpy(offs).to(DEV)
    BQ = F.query_tile_rows(h_q, h_kv, d)
    assert N // BQ + n > 12288
    need = F.ring_attn_workspace_bytes(N, N, h_q, h_kv, d, 1, True, n, True, F.BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    F.ring_attn_fwd(q, k, v, causal=True, seq_offsets=offs_d, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)
    n_items = int(w[0])
    ref_items, ref_n = F.jagged_worklist(offs_d, N, BQ)
    torch.cuda.synchronize()
    assert n_items == int(ref_n.item())
    assert np.array_equal(w[64:64 + 8 * n_items].reshape(n_items, 8), ref_items[:n_items].cpu().numpy())


@pytest.mark.parametrize("n_short", [3, 2100])
def test_prepass_sequence_beyond_1024_tiles(n_short):
    """One sequence of more than 1024 query tiles: the ranking by tile count
    puts it in the histogram's top bin, which both pre-pass paths order by an
    exact second pass.  With 3 short sequences the fused kernel runs, with 2100
    the two-kernel path; either way the records equal fakv_jagged_worklist's and
    every (record, head group) entry is queued once."""
    h_q = h_kv = 1
    d = 64
    BQ = F.query_tile_rows(h_q, h_kv, d)
    long_len = 1030 * BQ + 17                  # 1031 tiles
    lens = np.array([5] * (n_short // 2) + [long_len, 2 * BQ + 1] + [1] * (n_short - n_short // 2), dtype=np.int64)
    offs = seq_offsets_from_lengths(lens)
    N, n = int(offs[-1]), len(lens)
    q, k, v = (torch.zeros((N, h, d), dtype=torch.bfloat16, device=DEV) for h in (h_q, h_kv, h_kv))
    offs_d = torch.from_numpy(offs).to(DEV)
    need = F.ring_attn_workspace_bytes(N, N, h_q, h_kv, d, 1, True, n, True, F.BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    F.ring_attn_fwd(q, k, v, causal=True, seq_offsets=offs_d, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)
    n_items = int(w[0])
    ref_items, ref_n = F.jagged_worklist(offs_d, N, BQ)
    torch.cuda.synchronize()
    assert n_items == int(ref_n.item()) == int(sum((L + BQ - 1) // BQ for L in lens))
    assert np.array_equal(w[64:64 + 8 * n_items].reshape(n_items, 8), ref_items[:n_items].cpu().numpy())
    cap = N // BQ + n
    n_hg = h_q // (256 // BQ)
    o_sched = (256 + _a256(cap * 32) + _a256(cap * 4) + _a256((n + 1) * 4) + _a256(n * 4)) // 4
    stride = cap * n_hg
    qlen = w[16:24]
    entries = np.concatenate([w[o_sched + x * stride:o_sched + x * stride + int(qlen[x])] for x in range(8)])
    assert np.array_equal(np.sort(entries), np.arange(n_items * n_hg))
    # the long sequence is ranked first: its unit heads queue 0, longest query tile first
    first = w[o_sched] // n_hg
    assert w[64 + 8 * first] == n_short // 2 and w[64 + 8 * first + 1] == 1030

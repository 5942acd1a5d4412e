"""Flattened (sequence, query-tile) worklist of a jagged batch (CPU, exact ints).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "[pallas] Support dependent Tile.end bounds in Pallas", section
"Flattened worklists": every work item carries the resident source range of
its sequence (start and length) and the compact extent of its query tile
(start and extent); the compute end is the smaller of the source end and the
compact end, and it alone sets the KV trip count, while the full range sets
what stays resident.  The per-sequence KV end comes from the prefix offsets
(the reviewer's note on the same page: the jagged end is read from
seq_offsets[seq_idx + 1]).

Readings of what the page leaves open:
* One item per (sequence, query tile of BQ rows); a sequence of length L has
  ceil(L / BQ) tiles and zero-length sequences have none.
* Order: longest compute extent first, as a load-balancing schedule: items
  sorted by descending tile index, ties by ascending sequence index.  The order
  is fixed so that a device-built worklist can be compared bit for bit.
* Record: int32 x 8 = (seq, tile, range_start, range_len, tile_start,
  tile_extent, compute_end, 0).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class WorkItem:
    seq: int
    tile: int
    range_start: int
    range_len: int
    tile_start: int
    tile_extent: int
    compute_end: int


def worklist_ref(seq_offsets, BQ: int):
    o = [int(x) for x in np.asarray(seq_offsets).tolist()]
    items = []
    for b in range(len(o) - 1):
        L = o[b + 1] - o[b]
        for t in range(-(-L // BQ)):
            range_start, range_len = o[b], L
            tile_start = o[b] + t * BQ
            tile_extent = min(BQ, L - t * BQ)
            source_end = range_start + range_len
            compact_end = tile_start + tile_extent
            items.append(WorkItem(b, t, range_start, range_len, tile_start, tile_extent,
                                  min(source_end, compact_end)))
    items.sort(key=lambda it: (-it.tile, it.seq))
    return items


def worklist_array_ref(seq_offsets, BQ: int) -> np.ndarray:
    """The worklist as an (n_items, 8) int32 array in record layout."""
    items = worklist_ref(seq_offsets, BQ)
    a = np.zeros((len(items), 8), dtype=np.int32)
    for n, it in enumerate(items):
        a[n, :7] = (it.seq, it.tile, it.range_start, it.range_len, it.tile_start,
                    it.tile_extent, it.compute_end)
    return a

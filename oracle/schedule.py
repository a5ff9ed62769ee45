"""Integer work-list enumeration of the jagged tile scheduler (CPU reference).

TEST INFRASTRUCTURE ONLY.

[GEM-MFU, Detailed notes: JFA] names persistent-kernel scheduling and
[GEM-MFU, Detailed notes: GDPA] software tile scheduling for jagged tensors;
the pages give no algorithm.  The work list this library uses is defined here
as plainly as possible so that the device-built list can be compared with it
bit for bit:

* A work item is one (sequence b, head h, tile t).  In the forward and dQ
  passes a tile is a block of ``bm`` query rows; in the dK/dV pass it is a
  block of ``bn`` key rows.
* The cost of an item is the number of blocks the kernel visits for it:
  forward / dQ -- the number of ``bn``-row key blocks, counted from key 0,
  up to the last key visible to any row of the query tile;
  dK/dV -- the number of ``bm``-row query blocks from the first query block
  holding a row that sees a key of the tile up to the last query block.
* Items are ordered longest first (cost descending), ties broken by (b, h, t)
  ascending: the longest-processing-time-first list order.

Visibility is the same as in ``attention.visible_mask``: every key of the
sequence, or, when causal, keys j <= i + (Lk - Lq).
"""

import numpy as np


def _lengths(q_offsets, kv_offsets):
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    return np.diff(qo), np.diff(ko)


def _ceil_div(a, b):
    return -(-a // b)


def fwd_tile_costs(q_offsets, kv_offsets, bm, bn, causal):
    """Per sequence, the list of (t, cost) for its query tiles (forward / dQ)."""
    lq, lk = _lengths(q_offsets, kv_offsets)
    out = []
    for b in range(len(lq)):
        tiles = []
        for t in range(_ceil_div(int(lq[b]), bm)):
            last_row = min((t + 1) * bm, int(lq[b])) - 1
            if causal:
                kv_end = min(int(lk[b]), max(0, last_row + int(lk[b]) - int(lq[b]) + 1))
            else:
                kv_end = int(lk[b])
            tiles.append((t, _ceil_div(kv_end, bn)))
        out.append(tiles)
    return out


def kv_tile_costs(q_offsets, kv_offsets, bm, bn, causal):
    """Per sequence, the list of (t, cost) for its key tiles (dK/dV pass)."""
    lq, lk = _lengths(q_offsets, kv_offsets)
    out = []
    for b in range(len(lq)):
        tiles = []
        nq_blocks = _ceil_div(int(lq[b]), bm)
        for t in range(_ceil_div(int(lk[b]), bn)):
            if causal:
                # first query row that sees key t*bn: i >= t*bn - (Lk - Lq)
                first_row = max(0, t * bn - (int(lk[b]) - int(lq[b])))
                cost = max(0, nq_blocks - first_row // bm) if first_row < lq[b] else 0
            else:
                cost = nq_blocks
            tiles.append((t, cost))
        out.append(tiles)
    return out


def worklist(tile_costs, heads):
    """Items (b, h, t, cost) sorted by cost descending, then (b, h, t)."""
    items = []
    for b, tiles in enumerate(tile_costs):
        for h in range(heads):
            for t, cost in tiles:
                items.append((b, h, t, cost))
    items.sort(key=lambda it: (-it[3], it[0], it[1], it[2]))
    return items

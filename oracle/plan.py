"""Per-expert tile rule and the tile list (the plan) built from expert offsets.

What the pages fix: the M tile of each expert should come from that expert's
own row count rather than from the total rows of the launch (humming PR
#129, intro and commit 1 "Row-major tile model"), because a fixed M128 tile
gives unevenly routed experts extra mostly empty tiles (45 tiles instead of
32 at M=512, same commit), while an expert whose rows fill M128 tiles
exactly should get exactly full tiles (same page, last note under the
tables).  Small experts go to a separate small-M schedule below a cutoff
found by a dense sweep (commit 2 "Small-expert seed tile").  The pages'
constants (M128/M176, the 96-row cutoff, rows + sqrt(rows)) belong to an
H200 kernel; the constants below belong to this library's two kernels.

Rule for an expert with ``rows`` routed rows (integer only):
  rows == 0          -> no tiles
  rows <= S_MAX      -> STREAM class: one m-tile, tile_m = ceil16(rows)
  rows >  S_MAX      -> MFMA class:   n_m = ceil(rows / T_MAX) tiles,
                        tile_m = ceil16(ceil(rows / n_m));
                        tile i covers rows [i*tile_m, min((i+1)*tile_m, rows))

Plan layout (int32): an 8-word header, then 4 words per m-tile.
  header: [status, m_tiles, stream_m_tiles, mfma_m_tiles,
           stream_items, mfma_items, padded_rows, total_rows]
  tile:   [expert, first_row, rows, tile_m | class << 16]
STREAM tiles come first, then MFMA tiles; each class is in (expert, i)
order.  A work item is one m-tile times one n-tile of the class's width;
stream_items = stream_m_tiles * ceil(N/TN_STREAM),
mfma_items   = mfma_m_tiles * ceil(N/TN_MFMA).
status: 0 ok, 1 offsets invalid (offsets[0] != 0 or decreasing),
        2 the caller's buffer holds fewer tiles than the plan has.
Test infrastructure only.
"""

from __future__ import annotations

import numpy as np

GRAN = 16          # m granularity: rows of one MFMA block
S_MAX = 64         # largest expert served by the weight-streaming class
T_MAX = 128        # largest m-tile of the MFMA class
TN_STREAM = 64     # n granularity by which the plan counts streaming work
TN_MFMA = 512      # n width of one MFMA work item

CLASS_NONE, CLASS_STREAM, CLASS_MFMA = 0, 1, 2
HEADER_WORDS = 8
TILE_WORDS = 4

STATUS_OK, STATUS_BAD_OFFSETS, STATUS_CAPACITY = 0, 1, 2

# the order in which the library reports its constants
PLAN_PARAMS = (GRAN, S_MAX, T_MAX, TN_STREAM, TN_MFMA, HEADER_WORDS, TILE_WORDS)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tile_rule(rows: int):
    """(class, tile_m, n_m) for one expert with ``rows`` rows."""
    if rows <= 0:
        return CLASS_NONE, 0, 0
    if rows <= S_MAX:
        return CLASS_STREAM, _ceil_div(rows, GRAN) * GRAN, 1
    n_m = _ceil_div(rows, T_MAX)
    tile_m = _ceil_div(_ceil_div(rows, n_m), GRAN) * GRAN
    return CLASS_MFMA, tile_m, n_m


def plan_ref(offsets, E: int, N: int, max_tiles=None) -> np.ndarray:
    """The plan as an int32 array (header + tiles) for the given offsets."""
    if hasattr(offsets, "detach"):
        offsets = offsets.detach().cpu().numpy()
    off = np.asarray(offsets, dtype=np.int64)
    hdr = np.zeros(HEADER_WORDS, dtype=np.int64)
    if off[0] != 0 or np.any(np.diff(off[: E + 1]) < 0):
        hdr[0] = STATUS_BAD_OFFSETS
        return hdr.astype(np.int32)
    tiles = {CLASS_STREAM: [], CLASS_MFMA: []}
    padded = 0
    for e in range(E):
        rows = int(off[e + 1] - off[e])
        cls, tile_m, n_m = tile_rule(rows)
        for i in range(n_m):
            r0 = i * tile_m
            r = min(tile_m, rows - r0)
            tiles[cls].append((e, int(off[e]) + r0, r, tile_m | (cls << 16)))
            padded += tile_m - r
    ns, nm = len(tiles[CLASS_STREAM]), len(tiles[CLASS_MFMA])
    hdr[1:8] = (ns + nm, ns, nm, ns * _ceil_div(N, TN_STREAM), nm * _ceil_div(N, TN_MFMA),
                padded, int(off[E]))
    body = tiles[CLASS_STREAM] + tiles[CLASS_MFMA]
    if max_tiles is not None and len(body) > max_tiles:
        hdr[0] = STATUS_CAPACITY
        body = body[:max_tiles]
    flat = np.array(body, dtype=np.int64).reshape(-1)
    return np.concatenate([hdr, flat]).astype(np.int32)

"""Routing histogram, exclusive-scan expert offsets and the stable row map.

Grouped-contiguous means the routed rows of each expert sit in one
contiguous block (humming PR #129, benchmark command, ``--gemm_type
grouped_contiguous``).  The planning step that builds such a layout keeps a
per-expert histogram and prefix arrays (MoonEP PR #38, background section),
and its outputs are required to match an independent reference exactly
(same page, correctness section).  The order of the slots inside one
expert's block is not stated anywhere; the reading taken here is the
textbook stable counting sort: slots keep their flat (token, k) order.

    counts[e]        = #{ (t, j) : ids[t, j] == e }
    offsets[0]       = 0,  offsets[e+1] = offsets[e] + counts[e]
    row_of_slot[t*k+j] = offsets[e] + #{ earlier flat slots with expert e }

Ids outside [0, E) are not counted and get row -1.  Test infrastructure only.
"""

from __future__ import annotations

import numpy as np


def route_ref(topk_ids, E: int):
    """Returns (counts int32 [E], offsets int32 [E+1], row_of_slot int32 [T*k])."""
    if hasattr(topk_ids, "detach"):
        topk_ids = topk_ids.detach().cpu().numpy()
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    row = np.full(ids.shape, -1, dtype=np.int64)
    vpos = np.nonzero(valid)[0]
    order = vpos[np.argsort(ids[vpos], kind="stable")]
    row[order] = np.arange(len(order))
    return counts.astype(np.int32), offsets.astype(np.int32), row.astype(np.int32)

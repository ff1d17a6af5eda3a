"""Values the pages print, kept as cited text fixtures under tests/golden/
(each file names its source), checked against the oracle and the synthetic
workloads."""

import os

import numpy as np

import synth
from oracle import plan_ref
from oracle import plan as oplan

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


def test_plan_exact_fit_matches_pages():
    rows = _rows("plan_exact_fit.txt")
    assert len(rows) == 2
    for tokens, top_k, E, per, tiles, tile_m, padded in (map(int, r) for r in rows):
        assert tokens * top_k // E == per
        off = np.arange(E + 1, dtype=np.int64) * per          # balanced routing
        p = plan_ref(off, E, 4096)
        hdr = p[: oplan.HEADER_WORDS]
        assert hdr[0] == oplan.STATUS_OK
        assert hdr[1] == tiles and hdr[3] == tiles            # all MFMA-class tiles
        assert hdr[6] == padded
        body = p[oplan.HEADER_WORDS:].reshape(-1, 4)
        assert np.all(body[:, 2] == tile_m) and np.all((body[:, 3] & 0xFFFF) == tile_m)


def test_workload_shapes_match_pages():
    rows = _rows("workload_shapes.txt")
    assert len(rows) == 7
    for name, E, top_k, T, N, K in rows:
        cfg = synth.CONFIGS[name]
        assert (cfg["E"], cfg["top_k"], cfg["T"], cfg["N"], cfg["K"]) == tuple(map(int, (E, top_k, T, N, K))), name

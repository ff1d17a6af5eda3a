"""Pins for the route and plan oracles.

Route: the textbook stable counting sort written as a plain Python loop,
plus invariants (counts sum, monotone offsets, bijection, order kept within
an expert).  Plan: brute-force enumeration of every row count up to 4096
against the properties the rule must have (tiles partition each expert's
rows exactly once, no empty tile, tile_m a multiple of 16 and at most the
class limit, padding bounds, exactly full tiles where rows fill them).
"""

import numpy as np
import pytest

from oracle import plan as P
from oracle import plan_ref, route_ref, tile_rule


def _route_loop(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for v in flat:
        if 0 <= v < E:
            counts[v] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    nxt = list(offsets[:E])
    rows = []
    for v in flat:
        if 0 <= v < E:
            rows.append(nxt[v])
            nxt[v] += 1
        else:
            rows.append(-1)
    return counts, offsets, rows


@pytest.mark.parametrize("seed,T,k,E", [(0, 32, 2, 8), (1, 64, 8, 32), (2, 7, 3, 5),
                                        (3, 1, 1, 1), (4, 300, 4, 1000), (5, 0, 2, 4)])
def test_route_matches_counting_loop(seed, T, k, E):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    c, o, r = route_ref(ids, E)
    c2, o2, r2 = _route_loop(ids, E)
    assert list(c) == c2 and list(o) == o2 and list(r) == r2


def test_route_invariants_skewed_and_invalid():
    rng = np.random.default_rng(3)
    E = 16
    ids = np.minimum(rng.geometric(0.4, size=(500, 4)) - 1, E - 1).astype(np.int32)
    ids[7, 1] = -1
    ids[9, 0] = E          # out of range: not counted
    c, o, r = route_ref(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert c.sum() == valid.sum() and o[0] == 0 and np.all(np.diff(o) >= 0)
    assert np.all(r[~valid] == -1)
    rv = r[valid]
    assert sorted(rv.tolist()) == list(range(int(valid.sum())))
    for e in range(E):
        pos = np.nonzero(flat == e)[0]
        assert np.all(np.diff(r[pos]) == 1)          # stable: flat order kept
        if len(pos):
            assert r[pos[0]] == o[e]
    c2, o2, r2 = _route_loop(ids, E)
    assert list(r) == r2


def test_route_all_to_one_expert():
    ids = np.full((10, 3), 2, dtype=np.int32)
    c, o, r = route_ref(ids, 4)
    assert list(c) == [0, 0, 30, 0] and list(o) == [0, 0, 0, 30, 30]
    assert list(r) == list(range(30))


def _check_tiles(rows):
    cls, tile_m, n_m = tile_rule(rows)
    if rows == 0:
        assert (cls, tile_m, n_m) == (P.CLASS_NONE, 0, 0)
        return
    assert tile_m % P.GRAN == 0 and tile_m > 0
    if rows <= P.S_MAX:
        assert cls == P.CLASS_STREAM and n_m == 1 and tile_m - P.GRAN < rows <= tile_m
        return
    assert cls == P.CLASS_MFMA and tile_m <= P.T_MAX
    covered = []
    for i in range(n_m):
        r0 = i * tile_m
        r = min(tile_m, rows - r0)
        assert r > 0                                   # no empty tile
        covered.extend(range(r0, r0 + r))
    assert covered == list(range(rows))                # exact partition
    assert n_m == -(-rows // P.T_MAX)                  # fewest tiles of the class limit
    assert n_m * tile_m - rows < P.GRAN * n_m + tile_m  # padding bound


def test_tile_rule_every_row_count():
    for rows in range(0, 4097):
        _check_tiles(rows)


def test_tile_rule_exact_fit():
    # an expert whose rows fill T_MAX tiles exactly gets exactly full tiles
    for n in range(1, 40):
        cls, tile_m, n_m = tile_rule(n * P.T_MAX)
        assert (tile_m, n_m) == (P.T_MAX, n)
    # an expert just past one full tile gets two balanced tiles, not a full
    # tile plus a nearly empty one
    assert tile_rule(P.T_MAX + 2) == (P.CLASS_MFMA, -(-(P.T_MAX // 2 + 1) // P.GRAN) * P.GRAN, 2)


def test_plan_layout_and_stats():
    rng = np.random.default_rng(5)
    E, N = 32, 4096
    counts = rng.integers(0, 400, size=E)
    counts[[3, 9]] = 0
    counts[4] = 64
    counts[5] = 65
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    plan = plan_ref(off, E, N)
    hdr, body = plan[:8], plan[8:].reshape(-1, 4)
    assert hdr[0] == 0 and hdr[1] == len(body) == hdr[2] + hdr[3]
    assert hdr[4] == hdr[2] * -(-N // P.TN_STREAM) and hdr[5] == hdr[3] * -(-N // P.TN_MFMA)
    assert hdr[7] == off[-1]
    cls = body[:, 3] >> 16
    assert np.all(cls[: hdr[2]] == P.CLASS_STREAM) and np.all(cls[hdr[2]:] == P.CLASS_MFMA)
    seen = np.zeros(off[-1], dtype=np.int32)
    padded = 0
    for e, r0, r, tm in body:
        tm &= 0xFFFF
        assert off[e] <= r0 and r0 + r <= off[e + 1]
        seen[r0:r0 + r] += 1
        padded += tm - r
    assert np.all(seen == 1) and padded == hdr[6]
    for part in (body[: hdr[2]], body[hdr[2]:]):
        keys = [(int(e), int(r0)) for e, r0, _, _ in part]
        assert keys == sorted(keys)


def test_plan_bad_offsets_and_capacity():
    assert plan_ref(np.array([1, 2, 3]), 2, 256)[0] == P.STATUS_BAD_OFFSETS
    assert plan_ref(np.array([0, 5, 3]), 2, 256)[0] == P.STATUS_BAD_OFFSETS
    full = plan_ref(np.array([0, 300, 301]), 2, 256)
    capped = plan_ref(np.array([0, 300, 301]), 2, 256, max_tiles=2)
    assert capped[0] == P.STATUS_CAPACITY and full[1] == -(-300 // P.T_MAX) + 1
    assert np.array_equal(capped[8:], full[8:16])
    empty = plan_ref(np.zeros(9, dtype=np.int32), 8, 256)
    assert list(empty) == [0] * 8

"""Pins for oracle.csla (the CSLA mask): hand-derived fixtures, an independent
closed form over every workload geometry, special cases and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import csla, geometry as G
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, TINY_SIDES, workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "csla_hand.json")


def _interval_gap_mask(sides, q, t, n_sink, radius):
    """Second route: the projected query tile is an interval of rows (the
    projection is monotone with steps <= 1 when h <= H), so the token rule holds
    for some pair iff the gap between that interval and the key tile's rows is
    <= r in both axes."""
    H = sides[q]
    nbq = G.tiles_per_side(H, t)
    out = []
    for i in range(nbq):
        for j in range(nbq):
            row = []
            for s in range(q + 1):
                h = sides[s]
                nb = G.tiles_per_side(h, t)
                for a in range(nb):
                    for b in range(nb):
                        def gap(qi, ka):
                            lo = (qi * t * h) // H
                            hi = ((qi * t + min(t, H - qi * t) - 1) * h) // H
                            k_lo, k_hi = ka * t, min(ka * t + t, h) - 1
                            return max(0, k_lo - hi, lo - k_hi)
                        dist = max(gap(i, a), gap(j, b))
                        row.append(s < n_sink or (radius[s] >= 0 and dist <= radius[s]))
            out.append(row)
    return np.array(out)


def test_hand_fixture():
    fx = json.load(open(GOLDEN))
    g = fx["geometry"]
    for case in fx["cases"]:
        if case["budget"] > 0:
            m = csla.budget_mask(g["sides"], g["q_scale"], g["tile"], case["n_sink"], case["budget"])
        else:
            m = csla.block_mask(g["sides"], g["q_scale"], g["tile"], case["n_sink"], case["radius"])
        cnt, idx = csla.lists_from_mask(m)
        for q, want in case["lists"].items():
            q = int(q)
            assert list(idx[q, : cnt[q]]) == want, (case, q)


@pytest.mark.parametrize("sides,q,t,n_sink,r", [
    (TINY_SIDES, 4, 4, 3, 4), (TINY_SIDES, 4, 4, 3, 1), (TINY_SIDES, 4, 4, 0, 0),
    (SCHEDULE_13, 12, 8, 5, 2), (SCHEDULE_13, 12, 8, 5, 0), (SCHEDULE_13, 11, 8, 5, 2),
    (SCHEDULE_13, 10, 8, 5, 3), (SCHEDULE_13, 9, 8, 5, 2), (SCHEDULE_16, 15, 8, 5, 2),
    ((1, 3, 5, 7, 10), 4, 3, 1, 1), ((2, 5, 6, 9, 12), 4, 4, 2, 2),
])
def test_matches_interval_closed_form(sides, q, t, n_sink, r):
    radius = [r] * (q + 1)
    assert (csla.block_mask(sides, q, t, n_sink, radius) == _interval_gap_mask(sides, q, t, n_sink, radius)).all()


def test_mixed_radii_closed_form():
    sides, q, t = SCHEDULE_13, 12, 8
    radius = [-1, -1, 0, 1, 2, -1, 3, 0, 1, 4, 2, -1, 1]
    assert (csla.block_mask(sides, q, t, 2, radius) == _interval_gap_mask(sides, q, t, 2, radius)).all()


def test_special_cases():
    sides, q, t = SCHEDULE_13, 12, 8
    nqb, nkb, _, _ = G.counts(sides, q, t)
    tiles = G.key_tiles(sides, q, t)
    # a window wider than any grid keeps everything: dense
    assert csla.block_mask(sides, q, t, 0, [64] * 13).all()
    # every scale dropped: only the sink tiles remain
    m = csla.block_mask(sides, q, t, 5, [-1] * 13)
    sink = np.array([tl.scale < 5 for tl in tiles])
    assert (m == sink[None, :]).all()
    # no sink, only the query scale at radius 0: each query tile keeps exactly its own tile
    m = csla.block_mask(sides, q, t, 0, [-1] * 12 + [0])
    own = np.zeros((nqb, nkb), bool)
    base = nkb - nqb
    own[np.arange(nqb), base + np.arange(nqb)] = True
    assert (m == own).all()


def test_containment_sinks_and_own_tile():
    sides, q, t = SCHEDULE_13, 12, 8
    m = csla.block_mask(sides, q, t, 5, [2] * 13)
    nqb, nkb, _, _ = G.counts(sides, q, t)
    tiles = G.key_tiles(sides, q, t)
    sink = np.array([tl.scale < 5 for tl in tiles])
    assert m[:, sink].all()
    assert m[np.arange(nqb), nkb - nqb + np.arange(nqb)].all()


def test_tiny_tile_unit_reading_is_the_same_mask():
    """The small case's window 'radius 1 block in mapped coordinates' (key tile
    within one tile of the query tile's projected tile position) equals the
    4-token window here."""
    sides, q, t, n_sink = TINY_SIDES, 4, 4, 3
    H = sides[q]
    nbq = G.tiles_per_side(H, t)
    rows = []
    for i in range(nbq):
        for j in range(nbq):
            row = []
            for s in range(q + 1):
                nb = G.tiles_per_side(sides[s], t)
                pa, pb = (i * nb) // nbq, (j * nb) // nbq
                for a in range(nb):
                    for b in range(nb):
                        row.append(s < n_sink or max(abs(a - pa), abs(b - pb)) <= 1)
            rows.append(row)
    assert (np.array(rows) == csla.block_mask(sides, q, t, n_sink, [4] * 5)).all()


def test_budget_rows_are_radius_prefixes():
    """Sorting by admission radius first means the radius-r mask is a prefix of
    the budget ranking: a budget equal to a radius-r row's size keeps that row."""
    sides, q, t, n_sink = SCHEDULE_13, 11, 8, 5
    for r in (0, 1, 2):
        mr = csla.block_mask(sides, q, t, n_sink, [r] * (q + 1))
        for row in range(0, mr.shape[0], 7):
            k = int(mr[row].sum())
            mb = csla.budget_mask(sides, q, t, n_sink, k)
            assert (mb[row] == mr[row]).all()


def test_budget_counts_and_nesting():
    sides, q, t, n_sink = SCHEDULE_13, 11, 8, 5
    prev = None
    for k in (6, 11, 16, 27):
        m = csla.budget_mask(sides, q, t, n_sink, k)
        assert (m.sum(axis=1) == k).all()
        if prev is not None:
            assert (prev <= m).all()
        prev = m
    # floor: the sinks plus the query tile's own tile
    assert (csla.budget_mask(sides, q, t, n_sink, 1).sum(axis=1) == 6).all()


def test_lists_round_trip():
    m = csla.block_mask(TINY_SIDES, 4, 4, 3, [4] * 5)
    cnt, idx = csla.lists_from_mask(m)
    back = np.zeros_like(m)
    for r in range(m.shape[0]):
        assert (np.diff(idx[r, : cnt[r]]) > 0).all()
        assert (idx[r, cnt[r]:] == -1).all()
        back[r, idx[r, : cnt[r]]] = True
    assert (back == m).all()


@pytest.mark.parametrize("name,count,flop,kmin,kmean,kmax", [
    ("tiny_fp32", 0.4239, 0.4575, 11, 13.25, 16),
    ("last_scale_2b", 0.8250, 0.8431, 16, 30.09, 39),
    ("high_res_128", 0.9426, 0.9482, 19, 38.58, 48),
])
def test_workload_sparsity_figures(name, count, flop, kmin, kmean, kmax):
    """Block sparsity of the workloads' masks against figures derived
    independently of this oracle (a separate token-level brute force made
    when the workloads were specified; the pages print none for these
    shapes): count and token-weighted sparsity to 1e-4, kept tiles per row."""
    w = {x.name: x for x in W.ALL}[name]
    m = csla.block_mask(w.sides, w.q_scale, w.tile, w.n_sink, w.radii)
    c, f = csla.sparsity(m, w.sides, w.q_scale, w.tile)
    assert abs(c - count) < 1e-4 and abs(f - flop) < 1e-4
    k = m.sum(axis=1)
    assert (k.min(), k.max()) == (kmin, kmax) and abs(k.mean() - kmean) < 0.005


def test_side48_radius2_sparsity_figure():
    m = csla.block_mask(SCHEDULE_13, 11, 8, 5, [2] * 12)
    assert abs(csla.sparsity(m, SCHEDULE_13, 11, 8)[0] - 0.7467) < 1e-4

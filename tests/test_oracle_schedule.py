"""Pins of the per-scale loop oracle (no GPU).

Pinned by: the window schedule's radii for windows 3/5/7 (the pages' sizes,
radius = half the odd side); the join against Python set operations on the
lists; reductions of the whole loop to routes that do not use it: dense
scales equal torch's CPU scaled-dot-product attention, a window covering the
whole grid turns every joined scale into dense attention plus the upsampled
residual (that residual rebuilt from torch attention under the decision
scale's own lists and a per-token projection loop), an intersection with
such a window and a union with a sink-only window both give the CS4A lists
unchanged (the CS4A lists already hold every sink tile)."""
import numpy as np
import pytest
import torch

from oracle import cs4a as C
from oracle import csla as L
from oracle import geometry as G
from oracle import schedule as S
from varsparse_inputs import SCHEDULE_13, SpatialField

SIDES = (1, 2, 4, 8, 12, 16)
T, D, SINK = 4, 3, 2
B, H, DIM = 1, 2, 16


def test_window_radius_357():
    assert S.window_radius(13, 10) == [1] * 11
    assert S.window_radius(13, 11) == [2] * 12
    assert S.window_radius(13, 12) == [3] * 13
    assert S.window_radius(16, 15, (9,)) == [4] * 16
    for bad in ((13, 9, (3, 5, 7)), (13, 12, (3, 5, 4)), (13, 12, (0,)), (5, 5, (3,))):
        with pytest.raises(ValueError):
            S.window_radius(*bad)


def test_plan():
    p = S.plan(13, 9, 3)
    assert p == ["dense"] * 9 + ["decision"] + ["cs4a+csla"] * 3
    p = S.plan(16, 9, 3)
    assert p[10:13] == ["cs4a"] * 3 and p[13:] == ["cs4a+csla"] * 3
    assert S.plan(5, 4, 3) == ["dense"] * 4 + ["decision"]


@pytest.mark.parametrize("seed", range(4))
def test_join_matches_set_operations(seed):
    rng = np.random.default_rng(seed)
    a = rng.random((3, 5, 19)) < 0.3
    b = rng.random((5, 19)) < 0.4            # shared across the leading axis
    u, i = S.join_masks(a, b, "union"), S.join_masks(a, b, "intersection")
    for r in range(3):
        for q in range(5):
            sa, sb = set(np.flatnonzero(a[r, q])), set(np.flatnonzero(b[q]))
            assert set(np.flatnonzero(u[r, q])) == sa | sb
            assert set(np.flatnonzero(i[r, q])) == sa & sb
    cnt, idx = L.lists_from_mask(a)
    assert np.array_equal(S.mask_from_lists(cnt, idx), a)
    with pytest.raises(ValueError):
        S.join_masks(a, b, "xor")


def _inputs():
    f = SpatialField(0, 90, B, H, DIM)
    k, v = f.keys_values(SIDES, SINK)
    qs = [f.queries(s) for s in SIDES]
    return qs, k.astype(np.float64), v.astype(np.float64)


def _sdpa(q, k, v, keep=None):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    m = None if keep is None else torch.from_numpy(keep)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=DIM ** -0.5).numpy()


@pytest.fixture(scope="module")
def loop_full_window():
    qs, k, v = _inputs()
    return qs, k, v, S.scale_loop(qs, k, v, SIDES, T, D, SINK, 0.9, (33, 33), DIM ** -0.5)


def test_dense_scales_are_plain_attention(loop_full_window):
    qs, k, v, out = loop_full_window
    off = G.scale_offsets(SIDES)
    for q in range(D + 1):
        ref = _sdpa(qs[q], k[:, :, : off[q + 1]], v[:, :, : off[q + 1]])
        np.testing.assert_allclose(out[q]["o"], ref, rtol=0, atol=1e-10)


def test_full_window_gives_dense_plus_residual(loop_full_window):
    qs, k, v, out = loop_full_window
    off = G.scale_offsets(SIDES)
    nkD = off[D + 1]
    # the decision scale's block-sparse output rebuilt from its lists with torch
    tiles_d = G.key_tiles(SIDES, D, T)
    qt_d = G.query_tiles(SIDES, D, T)
    keep = np.zeros((B, H, SIDES[D] ** 2, nkD), bool)
    for b in range(B):
        for h in range(H):
            for i, qt in enumerate(qt_d):
                for j in out[D]["idx"][b, h, i, : out[D]["cnt"][b, h, i]]:
                    rows, cols = np.ix_(qt.tokens(), tiles_d[j].tokens())
                    keep[b, h, rows, cols] = True
    o_sparse_d = _sdpa(qs[D], k[:, :, :nkD], v[:, :, :nkD], keep)
    resid = _sdpa(qs[D], k[:, :, :nkD], v[:, :, :nkD]) - o_sparse_d
    for q in range(D + 1, len(SIDES)):
        nkb = len(G.key_tiles(SIDES, q, T))
        assert (out[q]["cnt"] == nkb).all()
        dense = _sdpa(qs[q], k[:, :, : off[q + 1]], v[:, :, : off[q + 1]])
        hd, ht = SIDES[D], SIDES[q]
        for y in range(ht):
            for x in range(ht):
                src = (y * hd // ht) * hd + (x * hd // ht)
                np.testing.assert_allclose(out[q]["o"][:, :, y * ht + x], dense[:, :, y * ht + x] + resid[:, :, src],
                                           rtol=0, atol=1e-10)
    assert np.abs(resid).max() > 1e-3    # the selection at D is a strict subset: the pin is not vacuous


@pytest.mark.parametrize("join,windows,override", [("intersection", (33, 33), None),
                                                   ("union", (3, 5), [-1] * len(SIDES))])
def test_joins_that_leave_cs4a_unchanged(join, windows, override):
    qs, k, v = _inputs()
    out = S.scale_loop(qs, k, v, SIDES, T, D, SINK, 0.9, windows, DIM ** -0.5, join=join, radius_override=override)
    scores = C.block_scores(qs[D], k, SIDES, D, T, DIM ** -0.5).astype(np.float32)
    sc, si = C.top_p_select(scores, 0.9)
    for q in range(D + 1, len(SIDES)):
        cnt, idx = C.map_indices(sc, si, SIDES, D, q, T, SINK)
        assert np.array_equal(out[q]["cnt"], cnt) and np.array_equal(out[q]["idx"], idx)


def test_union_contains_both_and_shrinks_with_window():
    qs, k, v = _inputs()
    u = S.scale_loop(qs, k, v, SIDES, T, D, SINK, 0.9, (3, 5), DIM ** -0.5)
    x = S.scale_loop(qs, k, v, SIDES, T, D, SINK, 0.9, (3, 5), DIM ** -0.5, join="intersection")
    for q in range(D + 1, len(SIDES)):
        win = L.block_mask(SIDES, q, T, SINK, S.window_radius(len(SIDES), q, (3, 5)))
        mu, mx = S.mask_from_lists(u[q]["cnt"], u[q]["idx"]), S.mask_from_lists(x[q]["cnt"], x[q]["idx"])
        assert (mu >= win).all() and (mx <= win).all() and (mx <= mu).all()
        assert mu.sum() > mx.sum()


def test_sink_tiles_in_every_sparse_list():
    """With a selection too small to reach the sinks on its own (top_p 0.05),
    every sparse scale of the loop, the decision scale included, still lists
    every sink tile (the sink region is appended to the mapped selection)."""
    qs, k, v = _inputs()
    out = S.scale_loop(qs, k, v, SIDES, T, D, SINK, 0.05, (3, 5), DIM ** -0.5)
    for q in range(D, len(SIDES)):
        tiles = G.key_tiles(SIDES, q, T)
        sinks = {j for j, tl in enumerate(tiles) if tl.scale < SINK}
        cnt, idx = out[q]["cnt"], out[q]["idx"]
        for row in range(cnt.shape[-1]):
            kept = set(idx[0, 0, row, : cnt[0, 0, row]].tolist())
            assert sinks <= kept
    # not vacuous: some decision rows select fewer than all sink tiles
    scores = C.block_scores(qs[D], k, SIDES, D, T, DIM ** -0.5).astype(np.float32)
    sel_cnt, sel_idx = C.top_p_select(scores, 0.05)
    tiles_d = G.key_tiles(SIDES, D, T)
    sinks_d = {j for j, tl in enumerate(tiles_d) if tl.scale < SINK}
    missing = [not sinks_d <= set(sel_idx[0, 0, r, : sel_cnt[0, 0, r]].tolist()) for r in range(sel_cnt.shape[-1])]
    assert any(missing)

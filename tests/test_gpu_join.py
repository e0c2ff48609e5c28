"""GPU parity: the join of kept-tile lists and the per-scale loop that uses it.

The join is integer work, so its lists must equal the oracle's bit for bit:
on seeded random lists (empty, full and partial rows; nkb below, at and
above a word and a wave of ids; one list set shared by every set), on lists
carrying entries the kernel must ignore, and at the full CS4A workload size
(B=2, H=16, targets 40/48/64, windows 3/5/7), where the joined lists must be
the union (or intersection) of the GPU's CS4A lists and the oracle's CSLA
window mask.  The loop itself (decision scale side 32: full and sparse
attention, scores, selection; each later scale: mapping, CSLA window mask,
union, block-sparse attention, O_cache correction) is compared with the
oracle two ways on two heads.  Stage by stage: each target's corrected output
against the oracle's block-sparse attention over the GPU's own joined lists,
corrected with the GPU's own decision-scale outputs, within the bf16 bar
2e-2.  End to end, against the oracle's loop from the inputs: lists
bit-exact, outputs within 6e-2, the sum of the bf16 output bound of the
three attention outputs entering each corrected value (the target's sparse
output, the decision scale's full and sparse outputs)."""
import math

import numpy as np
import pytest
import torch

from oracle import csla as L, cs4a as C, geometry as G, schedule as S
from tests._common import to_device
from varsparse_inputs import SpatialField, round_bf16, workloads as W

pytestmark = pytest.mark.gpu

WINDOWS = (3, 5, 7)
LOOP_TOL = 3 * 2e-2


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _random_lists(rng, lead, rows, nkb, density):
    m = rng.random((*lead, rows, nkb)) < density
    flat = m.reshape(-1, rows, nkb)
    flat[:, 0] = False                     # an empty row
    if rows > 1:
        flat[:, 1] = True                  # a full row
    return m, L.lists_from_mask(m)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


@pytest.mark.parametrize("join", ["union", "intersection"])
@pytest.mark.parametrize("nkb", [1, 31, 64, 172, 672, 5000, 65536])
@pytest.mark.parametrize("shared_b", [False, True])
def test_join_random_bit_exact(join, nkb, shared_b):
    vs = _vs()
    rng = np.random.default_rng(1000 + nkb + 7 * shared_b)
    rows = 17
    ma, (ac, ai) = _random_lists(rng, (3,), rows, nkb, 0.2)
    mb, (bc, bi) = _random_lists(rng, () if shared_b else (3,), rows, nkb, 0.3)
    oc, oi = vs.join_lists(_dev(ac), _dev(ai), _dev(bc), _dev(bi), join=join)
    torch.cuda.synchronize()
    ec, ei = L.lists_from_mask(S.join_masks(ma, mb, join))
    assert np.array_equal(oc.cpu().numpy(), ec)
    assert np.array_equal(oi.cpu().numpy(), ei)


def test_join_shared_a_and_both_shared():
    vs = _vs()
    rng = np.random.default_rng(7)
    ma, (ac, ai) = _random_lists(rng, (), 9, 100, 0.25)
    mb, (bc, bi) = _random_lists(rng, (2, 2), 9, 100, 0.25)
    oc, oi = vs.join_lists(_dev(ac), _dev(ai), _dev(bc), _dev(bi), join="union")
    ec, ei = L.lists_from_mask(S.join_masks(mb, ma, "union"))
    assert np.array_equal(oc.cpu().numpy(), ec) and np.array_equal(oi.cpu().numpy(), ei)
    _, (bc1, bi1) = _random_lists(rng, (), 9, 100, 0.25)
    oc, oi = vs.join_lists(_dev(ac), _dev(ai), _dev(bc1), _dev(bi1), join="intersection")
    ec, ei = L.lists_from_mask(S.join_masks(ma, S.mask_from_lists(bc1, bi1), "intersection"))
    assert np.array_equal(oc.cpu().numpy(), ec) and np.array_equal(oi.cpu().numpy(), ei)


def test_join_ignores_out_of_range_entries():
    """Ids outside [0, nkb) and counts outside [0, nkb] cannot move an access
    out of bounds: the ids are skipped and the counts clamped."""
    vs = _vs()
    nkb, rows = 40, 4
    ai = np.full((1, rows, nkb), -1, np.int32)
    bi = np.full((1, rows, nkb), -1, np.int32)
    ac = np.array([[3, 2, 50, -5]], np.int32)
    bc = np.array([[2, 3, 0, 2]], np.int32)
    ai[0, 0, :3] = [1, 40, 7]              # 40 is out of range
    ai[0, 1, :2] = [5, 9]
    ai[0, 2, :] = np.arange(nkb)           # count 50 > nkb: clamped to the whole row
    bi[0, 0, :2] = [7, -3]
    bi[0, 1, :3] = [9, 10, 1000]
    bi[0, 3, :2] = [0, 39]
    expect_u = [{1, 7}, {5, 9, 10}, set(range(nkb)), {0, 39}]
    expect_i = [{7}, {9}, set(), set()]
    for join, expect in (("union", expect_u), ("intersection", expect_i)):
        oc, oi = vs.join_lists(_dev(ac), _dev(ai), _dev(bc), _dev(bi), join=join)
        oc, oi = oc.cpu().numpy(), oi.cpu().numpy()
        for r in range(rows):
            assert oc[0, r] == len(expect[r])
            assert list(oi[0, r, : oc[0, r]]) == sorted(expect[r])
            assert (oi[0, r, oc[0, r]:] == -1).all()


@pytest.mark.parametrize("join", ["union", "intersection"])
def test_full_size_joined_lists(join):
    """The benchmarked shape: the GPU's CS4A lists of every target joined with
    the CSLA window lists; the result must be the set union/intersection of
    the GPU's CS4A lists and the oracle's window mask, row by row."""
    vs = _vs()
    w = W.CS4A
    D = W.CS4A_DECISION
    f = SpatialField(w.seed, w.wid, w.B, w.H, w.d)
    k, _ = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
    q_d = f.queries(w.sides[D])
    kd = to_device(k)
    scores, _, _, _, _ = vs.map_indices(w.sides, w.tile, D, D, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d), k=kd)
    n = len(w.sides)
    for T in W.CS4A_TARGETS:
        _, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores)
        radius = vs.window_radius(n, T, WINDOWS)
        mc, mi, _ = vs.build_mask(w.sides, w.tile, T, w.n_sink, radius=radius)
        jc, ji = vs.join_lists(kc, ki, mc, mi, join=join)
        torch.cuda.synchronize()
        win = L.block_mask(w.sides, T, w.tile, w.n_sink, S.window_radius(n, T, WINDOWS))
        assert np.array_equal(mc.cpu().numpy(), L.lists_from_mask(win)[0])
        cs4a = S.mask_from_lists(kc.cpu().numpy(), ki.cpu().numpy())
        ec, ei = L.lists_from_mask(S.join_masks(cs4a, win, join))
        assert np.array_equal(jc.cpu().numpy(), ec), T
        assert np.array_equal(ji.cpu().numpy(), ei), T


def test_scale_loop_stage_by_stage():
    """Each target scale's corrected output, given the GPU's own upstream
    results: the oracle's block-sparse attention over the GPU's joined lists,
    plus the nearest-upsampled residual of the GPU's decision-scale full and
    sparse outputs (the oracle's O_cache correction), within 2e-2; both as two
    launches (attention, then the correction) and as one."""
    from oracle import attention as OA, ocache as OO
    vs = _vs()
    w = W.CS4A
    D = W.CS4A_DECISION
    B, H = 1, 2
    n = len(w.sides)
    scale = 1 / math.sqrt(w.d)
    f = SpatialField(w.seed, w.wid, B, H, w.d)
    k, v = f.keys_values(w.sides, w.n_sink)
    k, v = round_bf16(k), round_bf16(v)
    qs = [round_bf16(f.queries(s)) for s in w.sides]
    off = G.scale_offsets(w.sides)
    kd, vd = to_device(k), to_device(v)
    qd = [to_device(x) for x in qs]
    nkD = off[D + 1]
    o_full, _ = vs.dense_attn_fwd(qd[D], kd[:, :, :nkD], vd[:, :, :nkD], softmax_scale=scale, want_lse=False)
    scores, _, _, dc, di = vs.map_indices(w.sides, w.tile, D, D, w.n_sink, W.CS4A_TOP_P, q_d=qd[D], k=kd)
    o_sparse, _ = vs.attn_fwd(qd[D], kd[:, :, :nkD], vd[:, :, :nkD], w.sides, w.tile, D, dc, di,
                              softmax_scale=scale, want_lse=False)
    of = o_full.float().cpu().numpy().astype(np.float64)
    osp = o_sparse.float().cpu().numpy().astype(np.float64)
    for T in W.CS4A_TARGETS:
        _, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores)
        mc, mi, _ = vs.build_mask(w.sides, w.tile, T, w.n_sink, radius=vs.window_radius(n, T, WINDOWS))
        jc, ji = vs.join_lists(kc, ki, mc, mi, join="union")
        nkT = off[T + 1]
        o, _ = vs.attn_fwd(qd[T], kd[:, :, :nkT], vd[:, :, :nkT], w.sides, w.tile, T, jc, ji,
                           softmax_scale=scale, want_lse=False)
        vs.ocache_correct(o_full, o_sparse, o, w.sides[D], w.sides[T])
        # the same step in one launch: the correction in the attention's epilogue
        o1, _ = vs.attn_fwd_ocache(qd[T], kd[:, :, :nkT], vd[:, :, :nkT], w.sides, w.tile, T, jc, ji, D, o_full,
                                   o_sparse, softmax_scale=scale, want_lse=False)
        torch.cuda.synchronize()
        ro, _ = OA.block_sparse_attention(qs[T], k[:, :, :nkT], v[:, :, :nkT], w.sides, T, w.tile,
                                          jc.cpu().numpy(), ji.cpu().numpy(), scale)
        want = OO.correct(ro, of, osp, w.sides[D], w.sides[T])
        err = np.abs(o.float().cpu().numpy() - want).max()
        assert err <= 2e-2, (T, err)
        err1 = np.abs(o1.float().cpu().numpy() - want).max()
        assert err1 <= 2e-2, (T, "one launch", err1)


def test_scale_loop_matches_oracle():
    vs = _vs()
    w = W.CS4A
    D = W.CS4A_DECISION
    B, H = 1, 2
    n = len(w.sides)
    scale = 1 / math.sqrt(w.d)
    f = SpatialField(w.seed, w.wid, B, H, w.d)
    k, v = f.keys_values(w.sides, w.n_sink)
    k, v = round_bf16(k), round_bf16(v)
    qs = [round_bf16(f.queries(s)) for s in w.sides]
    ref = S.scale_loop(qs, k, v, w.sides, w.tile, D, w.n_sink, W.CS4A_TOP_P, WINDOWS, scale)

    off = G.scale_offsets(w.sides)
    kd, vd = to_device(k), to_device(v)
    qd = [to_device(x) for x in qs]
    nkD = off[D + 1]
    o_full, _ = vs.dense_attn_fwd(qd[D], kd[:, :, :nkD], vd[:, :, :nkD], softmax_scale=scale, want_lse=False)
    scores, sc, si, dc, di = vs.map_indices(w.sides, w.tile, D, D, w.n_sink, W.CS4A_TOP_P, q_d=qd[D], k=kd,
                                           want_selection=True)
    o_sparse, _ = vs.attn_fwd(qd[D], kd[:, :, :nkD], vd[:, :, :nkD], w.sides, w.tile, D, dc, di,
                              softmax_scale=scale, want_lse=False)
    outs, lists = {}, {}
    for T in W.CS4A_TARGETS:
        _, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores)
        mc, mi, _ = vs.build_mask(w.sides, w.tile, T, w.n_sink, radius=vs.window_radius(n, T, WINDOWS))
        jc, ji = vs.join_lists(kc, ki, mc, mi, join="union")
        o, _ = vs.attn_fwd(qd[T], kd[:, :, : off[T + 1]], vd[:, :, : off[T + 1]], w.sides, w.tile, T, jc, ji,
                           softmax_scale=scale, want_lse=False)
        vs.ocache_correct(o_full, o_sparse, o, w.sides[D], w.sides[T])
        outs[T], lists[T] = o, (jc, ji)
    torch.cuda.synchronize()

    # decision rows whose selection differs from the oracle's own (float32
    # rounding of the scores at the top-p threshold) are excluded downstream;
    # there may be at most a few of them
    oc_sel, oi_sel = C.top_p_select(
        C.block_scores(qs[D], k, w.sides, D, w.tile, scale).astype(np.float32), W.CS4A_TOP_P)
    bad = (sc.cpu().numpy() != oc_sel) | (si.cpu().numpy() != oi_sel).any(-1)     # [B, H, nqb_D]
    assert bad.sum() <= max(1, bad.size // 50), f"{bad.sum()} decision rows differ"
    np.testing.assert_allclose(o_full.float().cpu().numpy(), ref[D]["o"], rtol=0, atol=2e-2)

    nbD = G.tiles_per_side(w.sides[D], w.tile)
    for T in W.CS4A_TARGETS:
        hT = w.sides[T]
        nbT = G.tiles_per_side(hT, w.tile)
        parent = np.array([(i // nbT * nbD // nbT) * nbD + (i % nbT * nbD // nbT) for i in range(nbT * nbT)])
        skip = bad[:, :, parent]                                                   # [B, H, nqb_T]
        jc, ji = (x.cpu().numpy() for x in lists[T])
        rc, ri = ref[T]["cnt"], ref[T]["idx"]
        assert np.array_equal(jc[~skip], rc[~skip]), T
        assert np.array_equal(ji[~skip], ri[~skip]), T
        # outputs: tokens whose tile list and whose O_cache source row are both unaffected
        got = outs[T].float().cpu().numpy()
        y, x = np.divmod(np.arange(hT * hT), hT)
        tile_of_tok = (y // w.tile) * nbT + x // w.tile
        hD = w.sides[D]
        src_tile = ((y * hD // hT) // w.tile) * nbD + (x * hD // hT) // w.tile
        for b in range(B):
            for h in range(H):
                ok = ~skip[b, h, tile_of_tok] & ~bad[b, h, src_tile]
                err = np.abs(got[b, h, ok] - ref[T]["o"][b, h, ok]).max()
                assert err <= LOOP_TOL, (T, b, h, err)

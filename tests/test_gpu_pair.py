"""GPU parity: block-sparse attention with 128-query workgroups over pairs of
query tiles (the block-128 variant).

Same bar as the 64-query kernel: bf16 outputs and lse within max-abs 2e-2 of
the float64 oracle on the same bf16 inputs.  Cases: the 2B-shaped last scale
with the CSLA lists (every tile, d = 128 and 64); an odd number of query
tiles (side 40: the last workgroup holds one tile); per-(b, h) random lists
with empty rows, full rows, rows that do not start at tile 0 and pairs whose
two lists differ; CS4A-mapped per-head lists; lists long enough that the
union walk rebuilds its chunk table (high-resolution geometry, full rows);
and the full-size 2B launch on sampled tiles, compared with the 64-query
kernel's output everywhere."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, geometry as G
from tests._common import gaussian, lists, oracle_mask, spatial, to_device
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, workloads as W

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _compare(o_gpu, lse_gpu, o_ref, lse_ref, where):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(o_ref[..., 0])
    err = np.abs(o - o_ref)[sel].max()
    assert err <= BF16_TOL, f"{where} max |O - O_ref| = {err}"
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lse_ref) & sel
    assert np.isneginf(lg[~np.isfinite(lse_ref) & sel]).all()
    if fin.any():
        assert np.abs(lg[fin] - lse_ref[fin]).max() <= BF16_TOL, where


@pytest.mark.parametrize("d", [128, 64])
def test_last_scale_every_tile(d):
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w, B=1, H=2)
    if d != w.d:
        q, k, v = q[..., :d].copy(), k[..., :d].copy(), v[..., :d].copy()
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o, lse = vs.attn_fwd_pair(to_device(q), to_device(k), to_device(v), w.sides, w.tile, w.q_scale, cnt, idx)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, f"pair last scale d={d}")


def test_odd_tile_count_and_partial_tiles():
    """Side 40 queries: 25 query tiles, so the last workgroup holds one tile;
    scales 3, 5, 12, 20 give partial key tiles."""
    vs = _vs()
    sides = (1, 2, 3, 5, 8, 12, 20, 24, 40)
    qs, t, d = 8, 8, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    assert nqb % 2 == 1
    q, k, v = gaussian(5, 51, 1, 2, nq, nk, d)
    radius = (2,) * 9
    cnt, idx, _ = vs.build_mask(sides, t, qs, 2, radius=radius)
    o, lse = vs.attn_fwd_pair(to_device(q), to_device(k), to_device(v), sides, t, qs, cnt, idx)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(sides, qs, t, 2, radius))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, mc, mi, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, "pair odd tile count")


def test_per_head_lists_that_differ_within_pairs():
    """Random per-(b, h) lists: empty rows (O = 0, lse = -inf), full rows,
    rows that skip tile 0, and every pair of tiles keeping different sets."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 11, 8
    B, H, d = 2, 2, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(21)
    keep = rng.random((B, H, nqb, nkb)) < rng.choice([0.05, 0.3, 0.7], size=(B, H, nqb, 1))
    keep[0, 0, 0] = False             # empty row paired with a non-empty one
    keep[0, 1, 1] = True              # full row
    keep[1, 0, 2] = False
    keep[1, 0, 2, 5:9] = True         # starts past tile 0
    keep[1, 1, 4:6] = False           # a whole pair empty
    cnt, idx = lists(keep)
    q, k, v = gaussian(6, 61, B, H, nq, nk, d)
    o, lse = vs.attn_fwd_pair(to_device(q), to_device(k), to_device(v), sides, t, qs,
                              torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, "pair per-head lists")
    o0 = o[0, 0, G.query_tiles(sides, qs, t)[0].tokens()].float()
    assert (o0 == 0).all()


def test_cs4a_lists():
    vs = _vs()
    w = W.CS4A
    D, T = W.CS4A_DECISION, W.CS4A_TARGETS[-1]
    q_d, k, v = spatial(w, B=1, H=2, q_side=w.sides[D])
    q_t = spatial(w, B=1, H=2, q_side=w.sides[T])[0]
    _, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d),
                                     k=to_device(k))
    o, lse = vs.attn_fwd_pair(to_device(q_t), to_device(k), to_device(v), w.sides, w.tile, T, kc, ki)
    torch.cuda.synchronize()
    ro, rl = OA.block_sparse_attention(q_t.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, T, w.tile, kc.cpu().numpy(), ki.cpu().numpy(), 1 / math.sqrt(w.d))
    _compare(o, lse, ro, rl, "pair cs4a lists")


def test_long_union_walk_rebuilds_the_table():
    """High-resolution geometry (672 key tiles): full rows make the union walk
    far longer than one chunk table; sampled query tiles compared."""
    vs = _vs()
    sides, qs, t = SCHEDULE_16, 15, 8
    B, H, d = 1, 1, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(31)
    keep = rng.random((B, H, nqb, nkb)) < 0.1
    keep[0, 0, 0:2] = True            # a pair of full rows: > 1300 chunks
    keep[0, 0, 2] = True
    keep[0, 0, 3] = False
    cnt, idx = lists(keep)
    q, k, v = gaussian(7, 71, B, H, nq, nk, d)
    o, lse = vs.attn_fwd_pair(to_device(q), to_device(k), to_device(v), sides, t, qs,
                              torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    tiles = [0, 1, 2, 3, 17, 100, 255]
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, 1 / math.sqrt(d), q_tiles=tiles)
    _compare(o, lse, ro, rl, "pair long union walk")


def test_full_size_matches_64_query_kernel_and_oracle():
    """The benchmarked launch (B=2, H=16, side 64 over 10521 tokens): the
    paired kernel's output equals the 64-query kernel's within the bf16 bar
    everywhere, and the oracle's on sampled (tile, head) pairs."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o1, l1 = vs.attn_fwd(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
    o2, l2 = vs.attn_fwd_pair(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= BF16_TOL
    assert (l1 - l2).abs().max().item() <= BF16_TOL
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(w.d),
                                       q_tiles=[0, 9, 36, 63], bh=[(0, 0), (1, 15)])
    _compare(o2, l2, ro, rl, "pair full size")

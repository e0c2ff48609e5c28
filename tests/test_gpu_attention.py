"""GPU parity: block-sparse and dense attention against the oracle.

Tolerances: bf16 outputs within max-abs 2e-2 of the float64 oracle on the
same bf16 inputs; fp32 outputs within 1e-4; lse alike."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, geometry as G
from tests._common import gaussian, lists, oracle_mask, spatial, to_device
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, round_bf16, workloads as W

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-4


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _compare(o_gpu, lse_gpu, o_ref, lse_ref, tol, where=""):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(o_ref[..., 0])
    err = np.abs(o - o_ref)[sel].max()
    assert err <= tol, f"{where} max |O - O_ref| = {err}"
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy().astype(np.float64)
        fin = np.isfinite(lse_ref) & sel
        assert (np.isneginf(lg[~np.isfinite(lse_ref) & sel])).all()
        if fin.any():
            e2 = np.abs(lg[fin] - lse_ref[fin]).max()
            assert e2 <= tol, f"{where} max |lse - lse_ref| = {e2}"
    return err


def test_fp32_tiny_workload():
    vs = _vs()
    w = W.TINY
    nqb, nkb, nq, nk = G.counts(w.sides, w.q_scale, w.tile)
    q, k, v = gaussian(w.seed, w.wid, w.B, w.H, nq, nk, w.d, bf16=False)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o, lse = vs.attn_fwd(to_device(q, torch.float32), to_device(k, torch.float32), to_device(v, torch.float32),
                         w.sides, w.tile, w.q_scale, cnt, idx, softmax_scale=1 / math.sqrt(w.d))
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(w.d))
    _compare(o, lse, ro, rl, FP32_TOL, "tiny fp32")


@pytest.mark.parametrize("d", [128, 64])
def test_bf16_last_scale_every_tile(d):
    """The 2B-shaped last scale (side 64 over 10521 cached tokens), one batch
    and two heads, every query tile compared."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w, B=1, H=2)
    if d != w.d:
        q, k, v = q[..., :d].copy(), k[..., :d].copy(), v[..., :d].copy()
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o, lse = vs.attn_fwd(to_device(q), to_device(k), to_device(v), w.sides, w.tile, w.q_scale, cnt, idx)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, BF16_TOL, f"last scale d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_bf16_partial_tiles(d):
    """Scales whose sides are not multiples of the tile (3, 5, 12, 20) give
    partial key tiles; side 40 queries (5 x 5 tiles)."""
    vs = _vs()
    sides = (1, 2, 3, 5, 8, 12, 20, 24, 40)
    qs, t = 8, 8
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    q, k, v = gaussian(3, 31, 1, 2, nq, nk, d)
    radius = (2,) * 9
    cnt, idx, _ = vs.build_mask(sides, t, qs, 2, radius=radius)
    o, lse = vs.attn_fwd(to_device(q), to_device(k), to_device(v), sides, t, qs, cnt, idx)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(sides, qs, t, 2, radius))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, mc, mi, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, BF16_TOL, f"partial tiles d={d}")


def test_bf16_per_head_lists_empty_rows_and_dense_rows():
    """Per-(b,h) lists drawn at random: rows with no tile (O = 0, lse = -inf),
    rows with every tile, rows that do not start at tile 0, and rows longer
    than 64 entries (the list is read in windows of 64)."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 11, 8
    B, H, d = 2, 2, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(11)
    keep = rng.random((B, H, nqb, nkb)) < rng.choice([0.05, 0.3, 0.7], size=(B, H, nqb, 1))
    keep[0, 0, 0] = False
    keep[0, 1, 1] = True
    keep[1, 0, 2] = False
    keep[1, 0, 2, 5:9] = True
    keep[1, 1, :, :3] = True
    cnt, idx = lists(keep)
    q, k, v = gaussian(4, 41, B, H, nq, nk, d)
    o, lse = vs.attn_fwd(to_device(q), to_device(k), to_device(v), sides, t, qs,
                         torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, BF16_TOL, "per-head lists")
    o0 = o[0, 0, G.query_tiles(sides, qs, t)[0].tokens()].float()
    assert (o0 == 0).all()
    assert torch.isneginf(lse[0, 0, G.query_tiles(sides, qs, t)[0].tokens()]).all()


@pytest.mark.parametrize("nq,nk,d", [(300, 1000, 128), (64, 32, 128), (1, 1, 128), (130, 257, 64), (2304, 6425, 128)])
def test_bf16_dense(nq, nk, d):
    vs = _vs()
    q, k, v = gaussian(5, 51, 1, 2, nq, nk, d)
    o, lse = vs.dense_attn_fwd(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    ro, rl = OA.dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, BF16_TOL, f"dense {nq}x{nk} d={d}")


@pytest.mark.parametrize("B,H,nq,nk,d,spike", [(1, 8, 2560, 700, 64, 0.0), (2, 16, 576, 1497, 128, 0.0),
                                                (1, 2, 300, 1000, 128, 8.0), (1, 8, 2560, 700, 64, 48.0),
                                                (1, 2, 130, 1000, 64, 8.0)])
def test_bf16_dense_split_walks(B, H, nq, nk, d, spike):
    """Dense launches over few 64-query blocks walk each block's keys in 2 or 4
    contiguous ranges, one per wave pair, and merge the pairs (the grid sizes
    here take 2, 2, 4, 2 and 4 pairs).  A spike scales a few keys in the last
    range: by 8 the pair's running maximum is raised within its walk and sits
    far above the other pairs' at the merge; by 48 the pair's fast walk
    overflows and the workgroup redoes its walks in the exact form."""
    vs = _vs()
    q, k, v = gaussian(7, 71, B, H, nq, nk, d)
    if spike:
        rows = np.arange(nk * 7 // 8, nk * 7 // 8 + 5)
        k[:, :, rows] = round_bf16(k[:, :, rows] * spike)
    o, lse = vs.dense_attn_fwd(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    bh = [(0, 0), (B - 1, H - 1), (0, H // 2)]
    rows = [0, 1, 63, 64, 65, nq // 2, nq - 1]
    ro, rl = OA.dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 1 / math.sqrt(d),
                                q_rows=rows, bh=bh)
    _compare(o, lse, ro, rl, BF16_TOL, f"dense split {B}x{H}x{nq}x{nk} d={d} spike={spike}")


@pytest.mark.parametrize("nq,nk,d", [(100, 333, 64), (64, 64, 128)])
def test_fp32_dense(nq, nk, d):
    vs = _vs()
    q, k, v = gaussian(6, 61, 1, 2, nq, nk, d, bf16=False)
    o, lse = vs.dense_attn_fwd(to_device(q, torch.float32), to_device(k, torch.float32), to_device(v, torch.float32))
    torch.cuda.synchronize()
    ro, rl = OA.dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, FP32_TOL, f"fp32 dense {nq}x{nk}")


def test_non_contiguous_strides():
    """Q/K/V/O as views of larger buffers (token stride > head dim)."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    sides, qs, t = w.sides[:10], 9, 8
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    q, k, v = gaussian(7, 71, 1, 2, nq, nk, 128)
    big = lambda x: torch.cat([to_device(x), to_device(np.zeros_like(x))], dim=-1)[..., :128]  # noqa: E731
    qd, kd, vd = big(q), big(k), big(v)
    out = torch.zeros(1, 2, nq, 256, dtype=torch.bfloat16, device="cuda")[..., 64:192]
    cnt, idx, _ = vs.build_mask(sides, t, qs, 5, radius=(2,) * 10)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, t, qs, cnt, idx, out=out)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(tuple(sides), qs, t, 5, (2,) * 10))
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, mc, mi, 1 / math.sqrt(128))
    _compare(o, lse, ro, rl, BF16_TOL, "strided")


SAMPLE_TILES = [0, 7, 9, 27, 36, 56, 63]


def test_full_size_2b_last_scale_sampled_and_deterministic():
    """The benchmarked launch: B=2, H=16, d=128, side 64 over 10521 tokens."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o1, l1 = vs.attn_fwd(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
    o2, l2 = vs.attn_fwd(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    bh = [(0, 0), (1, 15), (0, 7), (1, 3)]
    ro, rl = OA.block_sparse_attention(q, k, v, w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(w.d),
                                       q_tiles=SAMPLE_TILES, bh=bh)
    _compare(o1, l1, ro, rl, BF16_TOL, "2B full size")
    # dense comparator on the same tensors, a few query rows
    od, ld = vs.dense_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 2047, 4095]
    rdo, rdl = OA.dense_attention(q, k, v, 1 / math.sqrt(w.d), q_rows=rows, bh=bh)
    _compare(od, ld, rdo, rdl, BF16_TOL, "2B dense full size")



def test_key_value_offsets_at_the_addressing_limit():
    """K and V rows as far apart as the bf16 kernels address: a token stride
    that puts the last cached row's last byte just below 2^31 bytes from its
    head's base (the per-head offsets are 32-bit), and a head stride that puts
    the second head's base past 2^31 bytes (64-bit base).  The last query
    tiles attend the last cached rows.  One more stride step is refused."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    B, H, d = 1, 2, w.d
    q, k, v = spatial(w, B=B, H=H)
    nk = k.shape[2]
    st = ((2**31 - 1 - 2 * d) // (2 * (nk - 1))) // 8 * 8
    assert (nk - 1) * st * 2 + 2 * d < 2**31 <= (nk - 1) * (st + 8) * 2 + 2 * d
    assert nk * st * 2 > 2**31

    def far(x):
        buf = torch.empty(B * H * nk * st, dtype=torch.bfloat16, device="cuda")
        view = buf.as_strided((B, H, nk, d), (H * nk * st, nk * st, st, 1))
        view.copy_(to_device(x))
        return view

    qd, kd, vd = to_device(q), far(k), far(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o, lse = vs.attn_fwd(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
    od, ld = vs.dense_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii)))
    bh = [(0, 0), (0, 1)]
    ro, rl = OA.block_sparse_attention(q, k, v, w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(d),
                                       q_tiles=[0, 7, 56, 62, 63], bh=bh)
    _compare(o, lse, ro, rl, BF16_TOL, "K/V offsets at the limit")
    rows = [0, 4031, 4095]
    rdo, rdl = OA.dense_attention(q, k, v, 1 / math.sqrt(d), q_rows=rows, bh=bh)
    _compare(od, ld, rdo, rdl, BF16_TOL, "dense, K/V offsets at the limit")
    wider = torch.empty(nk * (st + 8), dtype=torch.bfloat16, device="cuda").as_strided(
        (1, 1, nk, d), (nk * (st + 8), nk * (st + 8), st + 8, 1))
    with pytest.raises(vs.VarsparseError):
        vs.attn_fwd(qd[:, :1], wider, wider, w.sides, w.tile, w.q_scale, cnt, idx)
    del kd, vd, wider
    torch.cuda.empty_cache()

def test_full_size_high_res_sampled():
    """High-resolution stress: B=1, H=16, side 128 queries over 42521 tokens."""
    vs = _vs()
    w = W.HIGH_RES
    q, k, v = spatial(w)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o, lse = vs.attn_fwd(to_device(q), to_device(k), to_device(v), w.sides, w.tile, w.q_scale, cnt, idx)
    torch.cuda.synchronize()
    mask = oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, tuple(w.radii))
    assert (cnt.cpu().numpy() == mask.sum(1)).all()
    mc, mi = lists(mask)
    ro, rl = OA.block_sparse_attention(q, k, v, w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(w.d),
                                       q_tiles=[0, 15, 100, 137, 255], bh=[(0, 0), (0, 9), (0, 15)])
    _compare(o, lse, ro, rl, BF16_TOL, "high-res")


@pytest.mark.parametrize("w", [W.LAST_TWO_8B_48, W.LAST_TWO_8B_64], ids=lambda w: w.name)
def test_full_size_budget_sweep_sampled(w):
    """The budget-sweep shape (B=2, H=28: 56 heads, a launch whose workgroups
    fill the chip 3.5 times at side 64) at each budget of the sweep
    (75/85/90/95% block sparsity): sampled query tiles of first, middle and
    last heads against the oracle, on the oracle's own budget lists."""
    vs = _vs()
    q, k, v = spatial(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    nqb = (w.sides[w.q_scale] // w.tile) ** 2
    tiles = sorted({0, 5, nqb // 2, nqb - 1})
    bh = [(0, 0), (1, 13), (1, 27)]
    for budget in w.budgets:
        print(f"budget sweep {w.name} budget={budget}", flush=True)
        cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, budget=budget)
        o, lse = vs.attn_fwd(qd, kd, vd, w.sides, w.tile, w.q_scale, cnt, idx)
        torch.cuda.synchronize()
        mask = oracle_mask(tuple(w.sides), w.q_scale, w.tile, w.n_sink, None, budget)
        mc, mi = lists(mask)
        assert np.array_equal(cnt.cpu().numpy(), mc)
        ro, rl = OA.block_sparse_attention(q, k, v, w.sides, w.q_scale, w.tile, mc, mi, 1 / math.sqrt(w.d),
                                           q_tiles=tiles, bh=bh)
        _compare(o, lse, ro, rl, BF16_TOL, f"{w.name} budget {budget}")


@pytest.mark.parametrize("per_head", [True, False])
def test_bf16_eight_heads_every_tile(per_head):
    """B H = 8 (one head per XCD range), shared and per-head random lists of
    mixed densities: every query tile of every head computed and right."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 10, 8
    B, H, d = 2, 4, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(77)
    shape = (B, H, nqb, nkb) if per_head else (nqb, nkb)
    keep = rng.random(shape) < rng.choice([0.02, 0.2, 0.6], size=shape[:-1] + (1,))
    cnt, idx = lists(keep)
    q, k, v = gaussian(8, 81, B, H, nq, nk, d)
    o, lse = vs.attn_fwd(to_device(q), to_device(k), to_device(v), sides, t, qs,
                         torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, 1 / math.sqrt(d))
    _compare(o, lse, ro, rl, BF16_TOL, f"eight heads per_head={per_head}")


@pytest.mark.parametrize("gain", [4.0, 16.0])
def test_bf16_large_scores_lazy_rescale(gain):
    """Q and K scaled up (scores of hundreds, softmax rows dominated by a few
    keys and running maxima raised many times over a row): sparse and dense
    attention stay within the bf16 bar of the float64 oracle."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 10, 8
    B, H, d = 1, 2, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    q, k, v = gaussian(9, 91, B, H, nq, nk, d, bf16=False)
    from varsparse_inputs import round_bf16
    q, k, v = round_bf16(q * np.float32(gain)), round_bf16(k * np.float32(gain / 4)), round_bf16(v)
    cnt, idx, _ = vs.build_mask(sides, t, qs, 5, radius=(2,) * (qs + 1))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, t, qs, cnt, idx)
    od, lsed = vs.dense_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    mc, mi = lists(oracle_mask(sides, qs, t, 5, (2,) * (qs + 1)))
    scale = 1 / math.sqrt(d)
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, mc, mi, scale)
    _compare(o, lse, ro, rl, BF16_TOL, f"large scores sparse gain={gain}")
    rows = np.arange(0, nq, 37)
    rdo, rdl = OA.dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale, q_rows=rows)
    _compare(od, lsed, rdo, rdl, BF16_TOL, f"large scores dense gain={gain}")


@pytest.mark.parametrize("case", ["underflow", "overflow"])
def test_bf16_extreme_score_ranges_every_kernel(case):
    """Scores outside the fast softmax form's range, so that it hands over to
    the exact form.  underflow: every score of every row about -130 or lower
    in the log2 domain (all weights against the starting maximum 0 flush to
    zero); overflow: the keys of one query-scale tile score about 160 above
    the rest (weights past 2^127).  Sparse, dense and token-exact kernels
    against the float64 oracle."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 10, 8
    B, H, d = 1, 2, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(77)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    from varsparse_inputs import round_bf16
    q = 32.0 * u + 0.05 * rng.standard_normal((B, H, nq, d))
    k = rng.standard_normal((B, H, nk, d))
    if case == "underflow":
        k = k - 32.0 * u
    else:
        off = G.scale_offsets(sides)[qs]
        side = sides[qs]
        toks = [off + y * side + x for y in range(8, 16) for x in range(16, 24)]   # one query-scale tile
        k[:, :, toks] = 40.0 * u + 0.1 * rng.standard_normal((B, H, len(toks), d))
    v = rng.standard_normal((B, H, nk, d))
    q, k, v = round_bf16(q.astype(np.float32)), round_bf16(k.astype(np.float32)), round_bf16(v.astype(np.float32))
    cnt, idx, _ = vs.build_mask(sides, t, qs, 5, radius=(2,) * (qs + 1))
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, t, qs, cnt, idx)
    od, lsed = vs.dense_attn_fwd(qd, kd, vd)
    ot, lset = vs.attn_fwd_token(qd, kd, vd, sides, t, qs, 5, (2,) * (qs + 1), cnt, idx)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    q64, k64, v64 = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    mc, mi = lists(oracle_mask(sides, qs, t, 5, (2,) * (qs + 1)))
    ro, rl = OA.block_sparse_attention(q64, k64, v64, sides, qs, t, mc, mi, scale)
    _compare(o, lse, ro, rl, BF16_TOL, f"{case} sparse")
    rows = np.arange(0, nq, 29)
    rdo, rdl = OA.dense_attention(q64, k64, v64, scale, q_rows=rows)
    _compare(od, lsed, rdo, rdl, BF16_TOL, f"{case} dense")
    rto, rtl = OA.token_masked_attention(q64, k64, v64, sides, qs, t, 5, (2,) * (qs + 1), scale,
                                         q_tiles=range(0, nqb, 5))
    _compare(ot, lset, rto, rtl, BF16_TOL, f"{case} token-exact")


def test_odd_head_count_every_tile_all_list_kernels():
    """B=1, H=3: the dispatch order interleaves the work items of head pairs
    and ranks each head's query tiles by list length, so the last pair holds
    a single head.  Per-head random lists whose lengths differ from tile to
    tile (an empty row in the lone head, a full row): every query tile of
    every head against the oracle for the 64-query and the paired-tile
    kernels; token-exact attention over the shared CSLA lists, three heads."""
    vs = _vs()
    sides, qs, t = SCHEDULE_13, 10, 8            # side 40: 25 query tiles, 72 key tiles
    B, H, d = 1, 3, 128
    scale = 1 / math.sqrt(d)
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(41)
    keep = rng.random((B, H, nqb, nkb)) < rng.choice([0.05, 0.2, 0.5, 0.9], size=(B, H, nqb, 1))
    keep[0, 2, 3] = False
    keep[0, 0, 7] = True
    cnt, idx = lists(keep)
    q, k, v = gaussian(8, 81, B, H, nq, nk, d)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    q64, k64, v64 = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    ro, rl = OA.block_sparse_attention(q64, k64, v64, sides, qs, t, cnt, idx, scale)
    cd, idd = torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda()
    for name, fn in (("64-query", vs.attn_fwd), ("paired", vs.attn_fwd_pair)):
        print(f"odd heads: {name}", flush=True)
        o, lse = fn(qd, kd, vd, sides, t, qs, cd, idd)
        torch.cuda.synchronize()
        _compare(o, lse, ro, rl, BF16_TOL, f"odd heads {name}")
        assert (o[0, 2, G.query_tiles(sides, qs, t)[3].tokens()].float() == 0).all()
    n_sink, rad = 5, [2] * (qs + 1)
    mc, mi, _ = vs.build_mask(sides, t, qs, n_sink, radius=rad)
    o, lse = vs.attn_fwd_token(qd, kd, vd, sides, t, qs, n_sink, rad, mc, mi)
    torch.cuda.synchronize()
    ro, rl = OA.token_masked_attention(q64, k64, v64, sides, qs, t, n_sink, rad, scale)
    _compare(o, lse, ro, rl, BF16_TOL, "odd heads token-exact")


def test_more_than_64_tiles_per_head_every_tile():
    """Query side 96 (144 query tiles, 72 pairs: more than the 64 items per
    head the dispatch order ranks, so these heads keep the natural order),
    B=1, H=3, per-head random lists of varied lengths with an empty and a
    full row: every query tile of every head against the oracle for the
    64-query and the paired-tile kernels."""
    vs = _vs()
    sides, qs, t = (1, 2, 4, 8, 16, 32, 48, 64, 96), 8, 8
    B, H, d = 1, 3, 128
    scale = 1 / math.sqrt(d)
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    assert nqb == 144
    rng = np.random.default_rng(97)
    keep = rng.random((B, H, nqb, nkb)) < rng.choice([0.02, 0.08, 0.2], size=(B, H, nqb, 1))
    keep[0, 1, 5] = False
    keep[0, 2, 100] = True
    cnt, idx = lists(keep)
    q, k, v = gaussian(9, 91, B, H, nq, nk, d)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, scale)
    cd, idd = torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda()
    for name, fn in (("64-query", vs.attn_fwd), ("paired", vs.attn_fwd_pair)):
        print(f"144 tiles: {name}", flush=True)
        o, lse = fn(qd, kd, vd, sides, t, qs, cd, idd)
        torch.cuda.synchronize()
        _compare(o, lse, ro, rl, BF16_TOL, f"144 tiles {name}")


@pytest.mark.parametrize("growth,spike", [(0.0, False), (6.0, False), (0.0, True)])
def test_long_lists_split_the_walk(growth, spike):
    """High-resolution geometry (16 scales, 672 key tiles, 42521 tokens): rows
    far longer than one chunk table (a full row, one contiguous run of 1329
    chunks; every other tile, no run past tile 0; a random tenth; an empty
    row), so that the walk is split into several table builds and each split
    takes the pending product of its last chunk.  With growth, key norms rise
    along the cache (x 7 at its end), so that later chunks' weights run far
    above the running maximum and it is raised many times, also right at the
    splits.  With spike, the 32 keys of the full row's chunk 511 (the last of
    its first table build) are scaled by 8, so that most of that row's
    queries raise their maximum on exactly that chunk and the split's drain
    applies the pending rescale (57 of tile 0's 64 queries, replaying the
    rule on the CPU).  The token-masked dense baseline (no lists: every key
    tile, the token rule applied) walks the same long rows."""
    vs = _vs()
    sides, qs, t = SCHEDULE_16, 15, 8
    B, H, d = 1, 2, 128
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    rng = np.random.default_rng(41)
    keep = rng.random((B, H, nqb, nkb)) < 0.1
    keep[0, 0, 0] = True            # the whole cache: one run
    keep[0, 0, 1] = False
    keep[0, 0, 1, ::2] = True       # every other tile
    keep[0, 0, 2] = False           # empty
    keep[0, 1, 5] = True
    cnt, idx = lists(keep)
    q, k, v = gaussian(9, 73, B, H, nq, nk, d)
    if growth:
        k = round_bf16(k * (1.0 + growth * np.arange(nk) / nk)[None, None, :, None])
    if spike:
        k = k.copy()
        k[:, :, 511 * 32: 512 * 32] *= 8.0
        k = round_bf16(k)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, t, qs, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    tiles = [0, 1, 2, 5, 100, 255]
    scale = 1 / math.sqrt(d)
    ro, rl = OA.block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       sides, qs, t, cnt, idx, scale, q_tiles=tiles)
    _compare(o, lse, ro, rl, BF16_TOL, f"long lists, growth {growth}, spike {spike}")
    n_sink, radius = 5, [2] * (qs + 1)
    ot, lt = vs.attn_fwd_token(qd, kd, vd, sides, t, qs, n_sink, radius)
    torch.cuda.synchronize()
    rto, rtl = OA.token_masked_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                         sides, qs, t, n_sink, radius, scale, q_tiles=[0, 37, 255])
    _compare(ot, lt, rto, rtl, BF16_TOL, f"token-masked dense, long rows, growth {growth}, spike {spike}")

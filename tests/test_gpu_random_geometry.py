"""GPU parity on seeded random geometries.

Each case draws a schedule of 3 to 8 strictly ascending scale sides (the
query scale last, its side a multiple of 8 up to 40; the earlier sides any
values below it, so key tiles are partial almost everywhere), a batch and
head count, a head dimension, a sink count and per-scale radii (some -1: the
scale dropped), or a budget; two more cases keep no sink and drop every
scale (every row empty) or all but the query scale's own window.  Checked on every query tile of every head:
the CSLA lists bit for bit against the oracle's mask; block-sparse attention
(64-query and paired-tile kernels), token-exact attention over the same
lists and dense attention against the oracle, outputs and lse within 2e-2;
and the fp32 kernel on random schedules with other tile sides (1e-4)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, csla as L, geometry as G
from tests._common import gaussian, to_device

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(3, 9))
    last = 8 * int(rng.integers(1, 6))
    sides = tuple(int(x) for x in np.sort(rng.choice(np.arange(1, last), size=n - 1, replace=False))) + (last,)
    q = n - 1
    n_sink = int(rng.integers(0, q + 1))
    radius = tuple(int(r) for r in rng.integers(-1, 4, size=n))
    budget = -1
    if seed % 4 == 3:
        nkb = G.counts(sides, q, 8)[1]
        budget = int(rng.integers(1, nkb + 1))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    if seed == 24:            # no sink, every scale dropped: every row empty
        n_sink, radius, budget = 0, (-1,) * n, -1
    if seed == 25:            # no sink, only the query scale's own tiles
        n_sink, radius, budget = 0, (-1,) * (n - 1) + (0,), -1
    return sides, q, n_sink, radius, budget, B, H, d


def _cmp(o, lse, ro, rl, where):
    og = o.float().cpu().numpy()
    err = np.abs(og - ro).max()
    assert err <= TOL, f"{where}: max |O - O_ref| = {err}"
    lg = lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert np.isneginf(lg[~fin]).all(), f"{where}: lse of empty rows"
    if fin.any():
        assert np.abs(lg[fin] - rl[fin]).max() <= TOL, f"{where}: lse"


@pytest.mark.parametrize("seed", range(26))
def test_random_geometry(seed):
    vs = _vs()
    sides, qs, n_sink, radius, budget, B, H, d = _draw(seed)
    where = f"seed {seed}: sides {sides} sink {n_sink} radius {radius} budget {budget} B {B} H {H} d {d}"
    print(where, flush=True)
    nqb, nkb, nq, nk = G.counts(sides, qs, 8)
    q, k, v = gaussian(300 + seed, 17, B, H, nq, nk, d)
    scale = 1.5 / math.sqrt(d)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    if budget > 0:
        cnt, idx, _ = vs.build_mask(sides, 8, qs, n_sink, budget=budget)
        mask = L.budget_mask(sides, qs, 8, n_sink, budget)
    else:
        cnt, idx, _ = vs.build_mask(sides, 8, qs, n_sink, radius=radius)
        mask = L.block_mask(sides, qs, 8, n_sink, list(radius))
    mc, mi = L.lists_from_mask(mask)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, 8, qs, cnt, idx, softmax_scale=scale)
    op, lsep = vs.attn_fwd_pair(qd, kd, vd, sides, 8, qs, cnt, idx, softmax_scale=scale)
    od, lsed = vs.dense_attn_fwd(qd, kd, vd, softmax_scale=scale)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), mc), where
    assert np.array_equal(idx.cpu().numpy(), mi), where
    q64, k64, v64 = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    ro, rl = OA.block_sparse_attention(q64, k64, v64, sides, qs, 8, mc, mi, scale)
    _cmp(o, lse, ro, rl, where + " (64-query kernel)")
    _cmp(op, lsep, ro, rl, where + " (paired-tile kernel)")
    rdo, rdl = OA.dense_attention(q64, k64, v64, scale)
    _cmp(od, lsed, rdo, rdl, where + " (dense)")
    if budget < 0:
        ot, lset = vs.attn_fwd_token(qd, kd, vd, sides, 8, qs, n_sink, radius, cnt, idx, softmax_scale=scale)
        torch.cuda.synchronize()
        rto, rtl = OA.token_masked_attention(q64, k64, v64, sides, qs, 8, n_sink, list(radius), scale)
        _cmp(ot, lset, rto, rtl, where + " (token-exact)")


@pytest.mark.parametrize("seed", range(10))
def test_random_geometry_fp32(seed):
    """The fp32 kernel (tiles of up to 64 tokens) on random schedules with
    tile sides 3, 4, 5 and 8: lists bit-exact, block-sparse and dense
    attention within 1e-4 of the oracle."""
    vs = _vs()
    rng = np.random.default_rng(9000 + seed)
    t = int(rng.choice([3, 4, 5, 8]))
    n = int(rng.integers(3, 7))
    last = t * int(rng.integers(max(1, -(-n // t)), 24 // t + 1))
    sides = tuple(int(x) for x in np.sort(rng.choice(np.arange(1, last), size=n - 1, replace=False))) + (last,)
    qs = n - 1
    n_sink = int(rng.integers(0, qs + 1))
    radius = tuple(int(r) for r in rng.integers(-1, 3, size=n))
    B, H, d = 1, int(rng.integers(1, 3)), int(rng.choice([64, 128]))
    where = f"seed {seed}: sides {sides} tile {t} sink {n_sink} radius {radius} H {H} d {d}"
    print(where, flush=True)
    nqb, nkb, nq, nk = G.counts(sides, qs, t)
    q, k, v = gaussian(500 + seed, 19, B, H, nq, nk, d, bf16=False)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = (to_device(x, torch.float32) for x in (q, k, v))
    cnt, idx, _ = vs.build_mask(sides, t, qs, n_sink, radius=radius)
    o, lse = vs.attn_fwd(qd, kd, vd, sides, t, qs, cnt, idx, softmax_scale=scale)
    od, lsed = vs.dense_attn_fwd(qd, kd, vd, softmax_scale=scale)
    torch.cuda.synchronize()
    mc, mi = L.lists_from_mask(L.block_mask(sides, qs, t, n_sink, list(radius)))
    assert np.array_equal(cnt.cpu().numpy(), mc), where
    assert np.array_equal(idx.cpu().numpy(), mi), where
    q64, k64, v64 = q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)
    ro, rl = OA.block_sparse_attention(q64, k64, v64, sides, qs, t, mc, mi, scale)
    rdo, rdl = OA.dense_attention(q64, k64, v64, scale)
    for (og, lg, rfo, rfl, what) in ((o, lse, ro, rl, "block-sparse"), (od, lsed, rdo, rdl, "dense")):
        err = np.abs(og.cpu().numpy() - rfo).max()
        assert err <= 1e-4, f"{where} ({what}): max |O - O_ref| = {err}"
        lgn = lg.cpu().numpy()
        fin = np.isfinite(rfl)
        assert np.isneginf(lgn[~fin]).all(), f"{where} ({what}): lse of empty rows"
        if fin.any():
            assert np.abs(lgn[fin] - rfl[fin]).max() <= 1e-4, f"{where} ({what}): lse"

"""GPU parity: token-exact CSLA attention (the token-level mask applied inside
the CSLA tiles) and the token-masked dense baseline (every key tile walked),
both against the oracle's attention under the token-level mask itself.

Tolerances as for the block-sparse kernel: bf16 outputs and lse within 2e-2
of the float64 oracle on the same bf16 inputs."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests._common import spatial, to_device
from varsparse_inputs import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _cmp(o, lse, ro, rl, where):
    og = o.float().cpu().numpy()
    sel = ~np.isnan(ro[..., 0])
    err = np.abs(og - ro)[sel].max()
    assert err <= TOL, f"{where}: max |O - O_ref| = {err}"
    lg = lse.cpu().numpy()
    fin = np.isfinite(rl) & sel
    assert np.isneginf(lg[~np.isfinite(rl) & sel]).all(), where
    assert np.abs(lg[fin] - rl[fin]).max() <= TOL, where


@pytest.mark.parametrize("n_sink,radius,d", [(5, 2, 128), (0, 1, 128), (3, 0, 64)])
def test_token_exact_and_token_dense_last_scale(n_sink, radius, d):
    """Side 64 over the 13-scale cache, one batch, two heads, every query
    tile; n_sink 0 exercises queries whose first walked chunks are fully
    masked."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w, B=1, H=2)
    if d != w.d:
        q, k, v = q[..., :d].copy(), k[..., :d].copy(), v[..., :d].copy()
    rad = [radius] * (w.q_scale + 1)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, n_sink, radius=rad)
    o1, l1 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, n_sink, rad, cnt, idx)
    o2, l2 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, n_sink, rad)
    torch.cuda.synchronize()
    ro, rl = OA.token_masked_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, n_sink, rad, scale)
    _cmp(o1, l1, ro, rl, f"token-exact sparse sink={n_sink} r={radius} d={d}")
    _cmp(o2, l2, ro, rl, f"token-masked dense sink={n_sink} r={radius} d={d}")


def test_dropped_scales_and_per_scale_radii():
    """Negative radii drop scales (sinks excepted); radii differ per scale."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w, B=1, H=1)
    rad = [0, 0, 0, 0, 0, -1, 1, -1, 2, 0, 3, 1, 2]
    n_sink = 2
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, n_sink, radius=rad)
    o1, l1 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, n_sink, rad, cnt, idx)
    o2, l2 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, n_sink, rad)
    torch.cuda.synchronize()
    ro, rl = OA.token_masked_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, n_sink, rad, 1 / math.sqrt(w.d))
    _cmp(o1, l1, ro, rl, "per-scale radii, sparse")
    _cmp(o2, l2, ro, rl, "per-scale radii, dense")


def test_token_exact_full_size_sampled():
    """The benchmarked shape (B=2, H=16): sampled query tiles of two heads
    against the oracle, for both walks."""
    vs = _vs()
    w = W.LAST_SCALE_2B
    q, k, v = spatial(w)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    cnt, idx, _ = vs.build_mask(w.sides, w.tile, w.q_scale, w.n_sink, radius=w.radii)
    o1, l1 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, w.n_sink, w.radii, cnt, idx)
    o2, l2 = vs.attn_fwd_token(qd, kd, vd, w.sides, w.tile, w.q_scale, w.n_sink, w.radii)
    torch.cuda.synchronize()
    tiles, bh = [0, 9, 35, 63], [(0, 3), (1, 15)]
    ro, rl = OA.token_masked_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                       w.sides, w.q_scale, w.tile, w.n_sink, w.radii, 1 / math.sqrt(w.d),
                                       q_tiles=tiles, bh=bh)
    _cmp(o1, l1, ro, rl, "full size sparse")
    _cmp(o2, l2, ro, rl, "full size dense")

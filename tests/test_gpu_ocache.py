"""GPU parity: the O_cache correction.

The kernel's fp32 arithmetic o + (f - p) on bf16 inputs, rounded once to
bf16, is compared with the oracle's float64 result rounded to bf16: they may
differ only by the double rounding (fp32 then bf16), i.e. at most one bf16
unit in the last place of the result (relative 2^-8) plus an absolute 1e-6
for results near zero.  Checked on random data at the decision/target sides
of the CS4A workload (32 -> 40, 48, 64, and 32 -> 32), head dims 64 and 128,
a non-contiguous target view, and end to end on the CS4A pipeline's own
outputs (decision scale full and sparse attention, target sparse attention).
The fused form (attention with the correction added before its one rounding)
is held to the oracle's exact attention plus the upsampled residual within
the bf16 output bar, its lse bit for bit to the attention's, and to the
two-call path within the second rounding the latter takes."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, ocache as OO
from tests._common import spatial, to_device
from varsparse_inputs import round_bf16, workloads as W

pytestmark = pytest.mark.gpu

ULP_REL = 2.0 ** -8
ABS_FLOOR = 1e-6


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _check(out, o_t, f, p, side_d, side_t, where):
    ref = round_bf16(OO.correct(o_t, f, p, side_d, side_t).astype(np.float32)).astype(np.float64)
    got = _bf16_np(out)
    err = np.abs(got - ref)
    bound = ULP_REL * np.abs(ref) + ABS_FLOOR
    assert (err <= bound).all(), f"{where}: {int((err > bound).sum())} values beyond one bf16 ulp, max {err.max()}"


@pytest.mark.parametrize("side_t", [32, 40, 48, 64])
@pytest.mark.parametrize("d", [128, 64])
def test_random_inputs(side_t, d):
    vs = _vs()
    rng = np.random.default_rng(100 + side_t + d)
    B, H, side_d = 2, 3, 32
    f = round_bf16(rng.normal(size=(B, H, side_d * side_d, d)).astype(np.float32)).astype(np.float64)
    p = round_bf16((f + 0.1 * rng.normal(size=f.shape)).astype(np.float32)).astype(np.float64)
    o_t = round_bf16(rng.normal(size=(B, H, side_t * side_t, d)).astype(np.float32)).astype(np.float64)
    out = to_device(o_t)
    vs.ocache_correct(to_device(f), to_device(p), out, side_d, side_t)
    torch.cuda.synchronize()
    _check(out, o_t, f, p, side_d, side_t, f"32->{side_t} d={d}")


def test_non_contiguous_target():
    """The target is a head-sliced view of a larger tensor (strides != sizes)."""
    vs = _vs()
    rng = np.random.default_rng(7)
    B, H, d, side_d, side_t = 1, 4, 128, 32, 48
    f = round_bf16(rng.normal(size=(B, H, side_d ** 2, d)).astype(np.float32)).astype(np.float64)
    p = round_bf16(rng.normal(size=f.shape).astype(np.float32)).astype(np.float64)
    big = round_bf16(rng.normal(size=(B, 2 * H, side_t ** 2, d)).astype(np.float32)).astype(np.float64)
    dev = to_device(big)
    view = dev[:, 1::2]
    vs.ocache_correct(to_device(f), to_device(p), view, side_d, side_t)
    torch.cuda.synchronize()
    _check(view, big[:, 1::2], f, p, side_d, side_t, "strided target")
    # the untouched heads are unchanged
    assert np.array_equal(_bf16_np(dev[:, 0::2]), big[:, 0::2])


def test_cs4a_pipeline_outputs():
    """End to end on the CS4A workload's shapes: full and block-sparse
    attention at the decision scale (its own selection, mapped D -> D), block-
    sparse attention at a target scale, then the correction."""
    vs = _vs()
    w = W.CS4A
    D, T = W.CS4A_DECISION, W.CS4A_TARGETS[0]
    B, H = 1, 2
    q_t, k, v = spatial(w, B=B, H=H)                 # cache of scales 0..12, queries at the last
    q_d = spatial(w, B=B, H=H, q_side=w.sides[D])[0]
    q_tt = spatial(w, B=B, H=H, q_side=w.sides[T])[0]
    nk_d = sum(s * s for s in w.sides[: D + 1])
    nk_t = sum(s * s for s in w.sides[: T + 1])
    kd, vd = to_device(k), to_device(v)
    _, _, _, cnt_d, idx_d = vs.map_indices(w.sides, w.tile, D, D, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d), k=kd)
    _, _, _, cnt_t, idx_t = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d), k=kd)
    qd_dev = to_device(q_d)
    o_full, _ = vs.dense_attn_fwd(qd_dev, kd[:, :, :nk_d], vd[:, :, :nk_d], want_lse=False)
    o_sparse, _ = vs.attn_fwd(qd_dev, kd, vd, w.sides, w.tile, D, cnt_d, idx_d, want_lse=False)
    o_t, _ = vs.attn_fwd(to_device(q_tt), kd, vd, w.sides, w.tile, T, cnt_t, idx_t, want_lse=False)
    torch.cuda.synchronize()
    before = _bf16_np(o_t)
    f, p = _bf16_np(o_full), _bf16_np(o_sparse)
    assert np.abs(f - p).max() > 0, "the decision-scale selection dropped nothing: no residual to test"
    vs.ocache_correct(o_full, o_sparse, o_t, w.sides[D], w.sides[T])
    torch.cuda.synchronize()
    _check(o_t, before, f, p, w.sides[D], w.sides[T], "cs4a pipeline")


def _ulp_bf16(x):
    """One bf16 unit in the last place of |x| (normal range)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


@pytest.mark.parametrize("ti,d", [(0, 128), (1, 128), (2, 128), (2, 64)])
def test_fused_attention_with_correction(ti, d):
    """varsparse_attn_fwd_ocache at the CS4A targets (sides 40, 48, 64) on the
    pipeline's own decision outputs and target lists."""
    vs = _vs()
    w = W.CS4A
    D, T = W.CS4A_DECISION, W.CS4A_TARGETS[ti]
    B, H = 1, 2
    q_t, k, v = spatial(w, B=B, H=H)
    if d != w.d:
        q_t, k, v = q_t[..., :d].copy(), k[..., :d].copy(), v[..., :d].copy()
    q_d = spatial(w, B=B, H=H, q_side=w.sides[D])[0][..., :d].copy()
    q_tt = spatial(w, B=B, H=H, q_side=w.sides[T])[0][..., :d].copy()
    nk_d = sum(s * s for s in w.sides[: D + 1])
    kd, vd, qd_dev, qt_dev = to_device(k), to_device(v), to_device(q_d), to_device(q_tt)
    _, outs = vs.map_indices_multi(w.sides, w.tile, D, [D, T], w.n_sink, W.CS4A_TOP_P, q_d=qd_dev, k=kd)
    (cnt_d, idx_d), (cnt_t, idx_t) = outs
    o_full, _ = vs.dense_attn_fwd(qd_dev, kd[:, :, :nk_d], vd[:, :, :nk_d], want_lse=False)
    o_sparse, _ = vs.attn_fwd(qd_dev, kd, vd, w.sides, w.tile, D, cnt_d, idx_d, want_lse=False)
    o_two, lse_two = vs.attn_fwd(qt_dev, kd, vd, w.sides, w.tile, T, cnt_t, idx_t)
    a_bf16 = o_two.clone()
    vs.ocache_correct(o_full, o_sparse, o_two, w.sides[D], w.sides[T])
    o_fused, lse_fused = vs.attn_fwd_ocache(qt_dev, kd, vd, w.sides, w.tile, T, cnt_t, idx_t, D, o_full, o_sparse)
    torch.cuda.synchronize()
    assert torch.equal(lse_fused, lse_two)
    f, p = _bf16_np(o_full), _bf16_np(o_sparse)
    assert np.abs(f - p).max() > 0, "the decision-scale selection dropped nothing: no residual to test"
    a_exact, _ = OA.block_sparse_attention(q_tt, k, v, w.sides, T, w.tile, cnt_t.cpu().numpy(), idx_t.cpu().numpy(),
                                           1 / math.sqrt(d))
    ref = OO.correct(a_exact, f, p, w.sides[D], w.sides[T])
    got, two, a = _bf16_np(o_fused), _bf16_np(o_two), _bf16_np(a_bf16)
    err = np.abs(got - ref).max()
    assert err <= 2e-2, f"fused vs oracle: {err}"
    # the two-call path rounds the attention to bf16 before the correction:
    # the results differ by at most that rounding plus each one's own
    bound = 0.5 * _ulp_bf16(a) + _ulp_bf16(np.maximum(np.abs(got), np.abs(two))) + ABS_FLOOR
    gap = np.abs(got - two)
    assert (gap <= bound).all(), f"fused vs two calls: {int((gap > bound).sum())} values, max {gap.max()}"

"""GPU parity: block-sparse attention of several query scales in one launch.

varsparse_attn_fwd_multi runs, per target, the walk of the one-target
kernels on the same inputs, so its outputs and lse must equal those of
attn_fwd (attn_fwd_ocache with the decision outputs) bit for bit: checked on
the CS4A targets (sides 40, 48, 64 over the 13-scale cache, per-(b, h) lists
mapped from decision side 32) at the benchmarked B = 2, H = 16, with and
without the O_cache correction, in either target order, at head dims 128 and
64, with shared CSLA lists over an odd number of heads (the last head pair
has one head), and for one and two targets.  One small case is also held to
the oracle's float64 block-sparse attention at the bf16 bar (2e-2)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, geometry as G
from tests._common import gaussian, spatial, to_device
from varsparse_inputs import workloads as W

pytestmark = pytest.mark.gpu


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _cs4a_inputs(B, H, d, seed):
    """Decision-scale queries, the cache of scales 0..12 and queries of every
    target (seeded Gaussian, bf16), with the CS4A lists of the targets."""
    vs = _vs()
    w = W.CS4A
    nk = G.scale_offsets(w.sides)[13]
    nq = {T: w.sides[T] ** 2 for T in (W.CS4A_DECISION,) + W.CS4A_TARGETS}
    q_all, k, v = gaussian(seed, 7, B, H, sum(nq.values()), nk, d)
    qs, off = {}, 0
    for T, n in nq.items():
        qs[T] = to_device(q_all[:, :, off:off + n].copy())
        off += n
    kd, vd = to_device(k), to_device(v)
    _, lists = vs.map_indices_multi(w.sides, w.tile, W.CS4A_DECISION, W.CS4A_TARGETS, w.n_sink, W.CS4A_TOP_P,
                                    q_d=qs[W.CS4A_DECISION], k=kd)
    return w, qs, kd, vd, dict(zip(W.CS4A_TARGETS, lists))


def _same(a, b, where):
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), where


@pytest.mark.parametrize("order", [(12, 11, 10), (10, 11, 12)])
@pytest.mark.parametrize("d", [128, 64])
def test_cs4a_targets_bit_identical(order, d):
    vs = _vs()
    w, qs, kd, vd, lists = _cs4a_inputs(2, 16, d, seed=31 + d)
    got = vs.attn_fwd_multi([qs[T] for T in order], kd, vd, w.sides, w.tile, order, [lists[T] for T in order])
    torch.cuda.synchronize()
    for T, (o, lse) in zip(order, got):
        ro, rl = vs.attn_fwd(qs[T], kd, vd, w.sides, w.tile, T, *lists[T])
        torch.cuda.synchronize()
        _same(o, ro, f"o of target {T}")
        _same(lse, rl, f"lse of target {T}")


def test_cs4a_targets_with_ocache_bit_identical():
    vs = _vs()
    w, qs, kd, vd, lists = _cs4a_inputs(2, 16, 128, seed=57)
    D = W.CS4A_DECISION
    rng = np.random.default_rng(5)
    shape = (2, 16, w.sides[D] ** 2, 128)
    f = torch.from_numpy(rng.normal(size=shape).astype(np.float32)).cuda().to(torch.bfloat16)
    p = (f.float() + 0.05 * torch.from_numpy(rng.normal(size=shape).astype(np.float32)).cuda()).to(torch.bfloat16)
    order = W.CS4A_TARGETS[::-1]
    got = vs.attn_fwd_multi([qs[T] for T in order], kd, vd, w.sides, w.tile, order, [lists[T] for T in order],
                            d_scale=D, o_full_d=f, o_sparse_d=p)
    torch.cuda.synchronize()
    for T, (o, lse) in zip(order, got):
        ro, rl = vs.attn_fwd_ocache(qs[T], kd, vd, w.sides, w.tile, T, *lists[T], D, f, p)
        torch.cuda.synchronize()
        _same(o, ro, f"o of target {T}")
        _same(lse, rl, f"lse of target {T}")


@pytest.mark.parametrize("targets", [(12, 10), (11,), (9, 12, 8)])
def test_shared_csla_lists_odd_heads(targets):
    """Shared CSLA lists (radius 2, sinks 0..4) over B = 1, H = 3: the last
    head pair holds one head; outputs of targets with and without lse."""
    vs = _vs()
    sides = W.LAST_SCALE_2B.sides
    nk = G.scale_offsets(sides)[max(targets) + 1]
    qs, lists = [], []
    for i, T in enumerate(targets):
        qs.append(to_device(gaussian(90 + i, 8, 1, 3, sides[T] ** 2, 1, 128)[0]))
        c, x, _ = vs.build_mask(sides, 8, T, 5, radius=[2] * (T + 1))
        lists.append((c, x))
    _, k, v = gaussian(80, 9, 1, 3, 1, nk, 128)
    kd, vd = to_device(k), to_device(v)
    lses = [None] + [torch.empty(1, 3, sides[T] ** 2, dtype=torch.float32, device="cuda") for T in targets[1:]]
    got = vs.attn_fwd_multi(qs, kd, vd, sides, 8, targets, lists, lses=lses)
    torch.cuda.synchronize()
    for T, q, (c, x), (o, lse) in zip(targets, qs, lists, got):
        ro, rl = vs.attn_fwd(q, kd, vd, sides, 8, T, c, x)
        torch.cuda.synchronize()
        _same(o, ro, f"o of target {T}")
        if lse is not None:
            _same(lse, rl, f"lse of target {T}")


def test_against_oracle():
    """Targets sides 40 and 48 (per-(b, h) CS4A lists) on spatially smooth
    inputs, B = 1, H = 2: every output against the oracle at 2e-2."""
    vs = _vs()
    w = W.CS4A
    D, targets = W.CS4A_DECISION, (11, 10)
    q_d, k, v = spatial(w, B=1, H=2, q_side=w.sides[D])
    kd, vd = to_device(k), to_device(v)
    _, lists = vs.map_indices_multi(w.sides, w.tile, D, targets, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d), k=kd)
    qs = {T: spatial(w, B=1, H=2, q_side=w.sides[T])[0] for T in targets}
    got = vs.attn_fwd_multi([to_device(qs[T]) for T in targets], kd, vd, w.sides, w.tile, targets, lists)
    torch.cuda.synchronize()
    for T, (c, x), (o, lse) in zip(targets, lists, got):
        nk = G.scale_offsets(w.sides)[T + 1]
        ro, rl = OA.block_sparse_attention(qs[T], k[:, :, :nk], v[:, :, :nk], w.sides, T, w.tile,
                                           c.cpu().numpy(), x.cpu().numpy(), 1 / math.sqrt(w.d))
        assert np.abs(o.float().cpu().numpy() - ro).max() <= 2e-2, T
        assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-2, T


def _dense_split(blocks: int, nk: int) -> bool:
    """Whether a one-target dense launch of this size splits each block's keys
    over wave pairs (the few-block form, which sums in another order)."""
    nch = (nk + 31) // 32
    return (blocks <= 256 and nch >= 24) or (blocks <= 512 and nch >= 12)


@pytest.mark.parametrize("d", [128, 64])
def test_dense_small_scales(d):
    """The scales below the CS4A decision scale (sides 1 ... 24), each over the
    cache of the scales up to its own, B = 2, H = 16, largest first and in
    ascending order.  Every output and lse equals dense_attn_fwd's bit for bit
    where that launch walks each 64-query block in one pass; where it splits
    a block's keys over wave pairs (few blocks), both are held to the
    oracle's float64 dense attention at 2e-2 on two heads."""
    vs = _vs()
    sides = W.CS4A.sides[:9]
    offs = G.scale_offsets(sides)
    B, H = 2, 16
    q_all, k, v = gaussian(61 + d, 10, B, H, int(offs[-1]), int(offs[-1]), d)
    kd, vd = to_device(k), to_device(v)
    qs = [to_device(q_all[:, :, offs[s]:offs[s + 1]].copy()) for s in range(len(sides))]
    nks = [int(offs[s + 1]) for s in range(len(sides))]
    bh = [(0, 0), (1, H - 1)]
    for order in (list(range(len(sides)))[::-1], list(range(len(sides)))):
        got = vs.dense_attn_fwd_multi([qs[s] for s in order], kd, vd, [nks[s] for s in order])
        torch.cuda.synchronize()
        for s, (o, lse) in zip(order, got):
            ro, rl = vs.dense_attn_fwd(qs[s], kd[:, :, : nks[s]], vd[:, :, : nks[s]])
            torch.cuda.synchronize()
            if not _dense_split(-(-sides[s] ** 2 // 64) * B * H, nks[s]):
                _same(o, ro, f"o of scale {s}")
                _same(lse, rl, f"lse of scale {s}")
                continue
            q = q_all[:, :, offs[s]:offs[s + 1]]
            xo, xl = OA.dense_attention(q, k[:, :, : nks[s]], v[:, :, : nks[s]], 1 / math.sqrt(d), bh=bh)
            for b, h in bh:
                for name, oo, ll in (("multi", o, lse), ("one-target", ro, rl)):
                    assert np.abs(oo[b, h].float().cpu().numpy() - xo[b, h]).max() <= 2e-2, (name, s, b, h)
                    assert np.abs(ll[b, h].cpu().numpy() - xl[b, h]).max() <= 2e-2, (name, s, b, h)


def test_dense_multi_against_oracle():
    """Three query sets (1, 100 and 300 queries: partial 64-query blocks) over
    cache prefixes of 7, 150 and 1000 keys, B = 1, H = 3, with and without
    lse: against the oracle's float64 dense attention at 2e-2."""
    vs = _vs()
    nqs, nks = (1, 100, 300), (7, 150, 1000)
    q_all, k, v = gaussian(71, 11, 1, 3, sum(nqs), max(nks), 128)
    kd, vd = to_device(k), to_device(v)
    qs, off = [], 0
    for n in nqs:
        qs.append(q_all[:, :, off:off + n].copy())
        off += n
    lses = [None] + [torch.empty(1, 3, n, dtype=torch.float32, device="cuda") for n in nqs[1:]]
    got = vs.dense_attn_fwd_multi([to_device(q) for q in qs], kd, vd, nks, lses=lses)
    torch.cuda.synchronize()
    for q, nk, (o, lse) in zip(qs, nks, got):
        ro, rl = OA.dense_attention(q, k[:, :, :nk], v[:, :, :nk], 1 / math.sqrt(128))
        assert np.abs(o.float().cpu().numpy() - ro).max() <= 2e-2, nk
        if lse is not None:
            assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-2, nk

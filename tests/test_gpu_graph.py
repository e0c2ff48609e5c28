"""GPU: the entry points under HIP graph capture.

The decision-scale and target-scale work of one generation step (dense
attention at the decision scale, CS4A scores with the select/map onto the
decision scale and three targets in one launch, block-sparse attention at the
decision scale, and per target the CSLA window lists, their union with the
CS4A lists and block-sparse attention with the O_cache correction) is
captured once in a graph on torch's capture stream.  The outputs are cleared
with eager fills between replays, other eager work runs between them, and
every replay must reproduce the eager step bit for bit (the kernels are
deterministic).  A second form runs the step as the scale loop of bench.py
does: the dense scales below the decision scale in one launch and the three
corrected target attentions in one launch.  Nothing the library does in a call is a memset or an
allocation, and the dynamic-LDS attributes are set before capture by the
eager step (once per kernel and device), so the graph holds kernels only."""
import math

import numpy as np
import pytest
import torch

from tests._common import to_device
from varsparse_inputs import SpatialField, round_bf16, workloads as W

pytestmark = pytest.mark.gpu


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


@pytest.mark.parametrize("several", [False, True], ids=["one_launch_per_scale", "several_scales_per_launch"])
def test_decision_and_target_scales_replay_in_a_graph(several):
    vs = _vs()
    w = W.CS4A
    D, targets = W.CS4A_DECISION, list(W.CS4A_TARGETS)
    B, H, d, t = 1, 2, w.d, w.tile
    n = len(w.sides)
    scale = 1 / math.sqrt(d)
    f = SpatialField(w.seed, w.wid, B, H, d)
    k, v = f.keys_values(w.sides, w.n_sink)
    kd, vd = to_device(round_bf16(k)), to_device(round_bf16(v))
    small = list(range(D))[::-1]
    qd = {s: to_device(round_bf16(f.queries(w.sides[s]))) for s in small + [D] + targets}
    nk = {s: vs.geom_counts(w.sides, t, s)[3] for s in small + [D] + targets}
    dev = kd.device

    def lists(s, lead):
        nqb, nkb = vs.geom_counts(w.sides, t, s)[:2]
        return (torch.empty(*lead, nqb, dtype=torch.int32, device=dev),
                torch.empty(*lead, nqb, nkb, dtype=torch.int32, device=dev))

    nqb_d, nkb_d = vs.geom_counts(w.sides, t, D)[:2]
    scores = torch.empty(B, H, nqb_d, nkb_d, dtype=torch.float32, device=dev)
    mapped = [lists(s, (B, H)) for s in [D] + targets]
    window = {T: lists(T, ()) for T in targets}
    joined = {T: lists(T, (B, H)) for T in targets}
    radius = {T: vs.window_radius(n, T, (3, 5, 7)) for T in targets}
    o_full, o_sparse = torch.empty_like(qd[D]), torch.empty_like(qd[D])
    outs = {T: torch.empty_like(qd[T]) for T in small + targets}

    def step():
        if several:
            vs.dense_attn_fwd_multi([qd[s] for s in small], kd, vd, [nk[s] for s in small], softmax_scale=scale,
                                    outs=[outs[s] for s in small], want_lse=False)
        vs.dense_attn_fwd(qd[D], kd[:, :, : nk[D]], vd[:, :, : nk[D]], softmax_scale=scale, out=o_full,
                          want_lse=False)
        vs.map_indices_multi(w.sides, t, D, [D] + targets, w.n_sink, W.CS4A_TOP_P, q_d=qd[D], k=kd,
                             softmax_scale=scale, scores=scores, out=mapped)
        vs.attn_fwd(qd[D], kd[:, :, : nk[D]], vd[:, :, : nk[D]], w.sides, t, D, *mapped[0], softmax_scale=scale,
                    out=o_sparse, want_lse=False)
        for i, T in enumerate(targets):
            vs.build_mask(w.sides, t, T, w.n_sink, radius=radius[T], out=(*window[T], None))
            vs.join_lists(*mapped[i + 1], *window[T], join="union", out=joined[T])
            if several:
                continue
            vs.attn_fwd_ocache(qd[T], kd[:, :, : nk[T]], vd[:, :, : nk[T]], w.sides, t, T, *joined[T], D, o_full,
                               o_sparse, softmax_scale=scale, out=outs[T], want_lse=False)
        if several:
            order = targets[::-1]
            vs.attn_fwd_multi([qd[T] for T in order], kd, vd, w.sides, t, order, [joined[T] for T in order],
                              softmax_scale=scale, outs=[outs[T] for T in order], want_lse=False, d_scale=D,
                              o_full_d=o_full, o_sparse_d=o_sparse)

    produced = [scores, o_full, o_sparse, *[x for pair in mapped for x in pair],
                *[x for T in targets for x in (*window[T], *joined[T], outs[T])]]
    if several:
        produced += [outs[s] for s in small]

    def snapshot():
        return [x.view(torch.int16) if x.dtype == torch.bfloat16 else x.clone() for x in produced]

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in snapshot()]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.empty_like(o_full)
    for r in range(3):
        for x in produced:
            x.fill_(0)
        vs.dense_attn_fwd(qd[D], kd[:, :, : nk[D]], vd[:, :, : nk[D]], out=other, want_lse=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(snapshot(), ref)):
            assert torch.equal(a, b), f"replay {r}: output {j} differs from the eager step"
    assert np.abs(o_full.float().cpu().numpy() - o_sparse.float().cpu().numpy()).max() > 0

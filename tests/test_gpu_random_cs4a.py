"""GPU parity of CS4A on seeded random geometries.

Each case draws a schedule of 4 to 9 strictly ascending sides whose last
three (the decision scale and two later targets) are multiples of 8 and the
earlier ones any values (partial key tiles), a sink count, a batch and head
count, a head dimension, a score sharpness and either top-p with a random p
or the Top-K rule with a random fraction.  One multi-target call scores the
decision scale and maps its selection onto itself and both targets; a
single-target call returns the selection.  Checked: scores within 1e-5 of the
oracle's (rows summing to 1); the selection and every target's lists bit for
bit against the oracle's select/map fed with the GPU's own scores."""
import math

import numpy as np
import pytest
import torch

from oracle import cs4a as OC, geometry as G
from tests._common import gaussian, to_device

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-5


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _draw(seed):
    rng = np.random.default_rng(11000 + seed)
    n_small = int(rng.integers(1, 7))
    d_side = 8 * int(rng.integers(2, 5))                         # 16 .. 32
    t1 = d_side + 8 * int(rng.integers(1, 3))
    t2 = t1 + 8 * int(rng.integers(1, 3))
    small = np.sort(rng.choice(np.arange(1, d_side), size=n_small, replace=False))
    sides = tuple(int(x) for x in small) + (d_side, t1, t2)
    D = n_small
    n_sink = int(rng.integers(0, D + 1))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    sharp = float(rng.choice([1.0, 3.0]))
    if seed % 3 == 2:
        rule, param = "top_k", float(rng.choice([0.05, 0.2, 0.5, 1.0]))
    else:
        rule, param = "top_p", float(rng.uniform(0.3, 1.0))
    return sides, D, n_sink, B, H, d, sharp, rule, param


@pytest.mark.parametrize("seed", range(12))
def test_random_cs4a(seed):
    vs = _vs()
    sides, D, n_sink, B, H, d, sharp, rule, param = _draw(seed)
    T1, T2 = D + 1, D + 2
    where = f"seed {seed}: sides {sides} D {D} sink {n_sink} B {B} H {H} d {d} sharp {sharp} {rule} {param:.3f}"
    print(where, flush=True)
    nqbD, nkbD, nqD, nkD = G.counts(sides, D, 8)
    q_d, k, _ = gaussian(700 + seed, 23, B, H, nqD, nkD, d)
    scale = sharp / math.sqrt(d)
    qd, kd = to_device(q_d), to_device(k)
    scores, outs = vs.map_indices_multi(sides, 8, D, [D, T1, T2], n_sink, param, rule=rule, q_d=qd, k=kd,
                                        softmax_scale=scale)
    sel_kw = dict(top_k=param) if rule == "top_k" else {}
    _, sc, si, _, _ = vs.map_indices(sides, 8, D, D, n_sink, param if rule == "top_p" else 0.9, scores=scores,
                                     want_selection=True, **sel_kw)
    torch.cuda.synchronize()
    s_gpu = scores.cpu().numpy()
    ref = OC.block_scores(q_d.astype(np.float64), k.astype(np.float64), sides, D, 8, scale)
    err = np.abs(s_gpu - ref).max()
    assert err <= SCORE_TOL, f"{where}: scores {err}"
    assert np.abs(s_gpu.astype(np.float64).sum(-1) - 1).max() < 1e-4, where
    if rule == "top_k":
        cnt, idx = OC.top_k_select(s_gpu, param)
    else:
        cnt, idx = OC.top_p_select(s_gpu, param)
    assert np.array_equal(sc.cpu().numpy(), cnt), f"{where}: selection counts"
    assert np.array_equal(si.cpu().numpy(), idx), f"{where}: selection ids"
    for T, (kc, ki) in zip((D, T1, T2), outs):
        mc, mi = OC.map_indices(cnt, idx, sides, D, T, 8, n_sink)
        assert np.array_equal(kc.cpu().numpy(), mc), f"{where}: lists of scale {T} (counts)"
        assert np.array_equal(ki.cpu().numpy(), mi), f"{where}: lists of scale {T} (ids)"

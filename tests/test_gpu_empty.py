"""GPU: empty inputs through the binding.  An empty batch (B == 0 or H == 0),
a dense call without queries and a join of no list sets return empty results
without an error and leave the device usable: a dense call right after still
matches the oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests._common import gaussian, to_device
from varsparse_inputs import SCHEDULE_13

pytestmark = pytest.mark.gpu

SIDES, T = SCHEDULE_13, 8


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


def _zeros(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype, device="cuda")


@pytest.mark.parametrize("B,H", [(0, 16), (2, 0)])
def test_empty_batch_every_entry_point(B, H):
    vs = _vs()
    qs, D = 10, 9
    nqb, nkb, nq, nk = vs.geom_counts(SIDES, T, qs)
    q, k, v = _zeros(B, H, nq, 128), _zeros(B, H, nk, 128), _zeros(B, H, nk, 128)
    cnt, idx, _ = vs.build_mask(SIDES, T, qs, 5, radius=[2] * (qs + 1))
    for fn in (vs.attn_fwd, vs.attn_fwd_pair):
        o, lse = fn(q, k, v, SIDES, T, qs, cnt, idx)
        assert o.shape == q.shape and lse.shape == (B, H, nq)
    o, lse = vs.attn_fwd_token(q, k, v, SIDES, T, qs, 5, [2] * (qs + 1))
    assert o.shape == q.shape
    o, lse = vs.dense_attn_fwd(q, k, v)
    assert o.shape == q.shape

    nqbD, nkbD, nqD, _ = vs.geom_counts(SIDES, T, D)
    q_d = _zeros(B, H, nqD, 128)
    scores, sc, si, kc, ki = vs.map_indices(SIDES, T, D, qs, 5, 0.9, q_d=q_d, k=k, want_selection=True)
    assert scores.shape == (B, H, nqbD, nkbD) and kc.shape == (B, H, nqb) and ki.shape == (B, H, nqb, nkb)
    scores, outs = vs.map_indices_multi(SIDES, T, D, [qs, 11], 5, 0.9, q_d=q_d, k=k)
    assert len(outs) == 2 and outs[0][0].shape == (B, H, nqb)

    nd = vs.geom_counts(SIDES, T, D)[2]
    f = _zeros(B, H, nd, 128)
    assert vs.ocache_correct(f, f.clone(), _zeros(B, H, nq, 128), SIDES[D], SIDES[qs]).shape == (B, H, nq, 128)

    ac = torch.zeros(B, H, nqb, dtype=torch.int32, device="cuda")
    ai = torch.zeros(B, H, nqb, nkb, dtype=torch.int32, device="cuda")
    oc, oi = vs.join_lists(ac, ai, cnt, idx)
    assert oc.shape == (B, H, nqb) and oi.shape == (B, H, nqb, nkb)
    torch.cuda.synchronize()
    _dense_still_right(vs)


def test_dense_without_queries():
    vs = _vs()
    q, k, v = _zeros(1, 2, 0, 128), _zeros(1, 2, 50, 128), _zeros(1, 2, 50, 128)
    o, lse = vs.dense_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)
    _dense_still_right(vs)


def _dense_still_right(vs):
    q, k, v = gaussian(3, 31, 1, 2, 70, 90, 128)
    o, lse = vs.dense_attn_fwd(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    ro, rl = OA.dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                1 / math.sqrt(128))
    assert np.abs(o.float().cpu().numpy() - ro).max() <= 2e-2
    assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-2

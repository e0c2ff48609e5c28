"""Shared helpers of the GPU parity tests: seeded inputs in the two forms
the two sides consume (bf16 device tensors for the HIP path, float64 arrays of
the same bf16 values for the oracle) and cached oracle masks."""
from __future__ import annotations

import functools

import numpy as np
import torch

from oracle import csla
from varsparse_inputs import SpatialField, bf16_bits, gaussian_qkv, round_bf16


def to_device(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    if dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.cuda()


def spatial(w, B=None, H=None, q_side=None, seed=None):
    """bf16-rounded float32 (q, k, v) of a workload, optionally shrunk."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    f = SpatialField(w.seed if seed is None else seed, w.wid, B, H, w.d)
    k, v = f.keys_values(w.sides[: w.q_scale + 1], w.n_sink, largest_side=w.sides[w.q_scale])
    q = f.queries(w.sides[w.q_scale] if q_side is None else q_side)
    return round_bf16(q), round_bf16(k), round_bf16(v)


def gaussian(seed, wid, B, H, nq, nk, d, bf16=True):
    q, k, v = gaussian_qkv(seed, wid, B, H, nq, nk, d)
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


@functools.lru_cache(maxsize=None)
def oracle_mask(sides, q_scale, t, n_sink, radius, budget=-1):
    if budget > 0:
        return csla.budget_mask(sides, q_scale, t, n_sink, budget)
    return csla.block_mask(sides, q_scale, t, n_sink, list(radius))


def lists(mask):
    return csla.lists_from_mask(mask)

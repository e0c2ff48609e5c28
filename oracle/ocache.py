"""O_cache: the decision scale's residual output, upsampled onto a later scale
to correct its sparse attention output (oracle; test infrastructure).

Source: SparVAR, ai.info summary, "Methodology in Plain English" (the first
module, CS4A) and "Main Findings" (the item on the two modules' increments).
In this implementation's terms: at the decision scale, the part of the full
attention output that the sparse selection misses is stored; it is enlarged
to each later scale's grid and added to that scale's sparse output (the
pages credit it with a PSNR gain at negligible cost).

Readings taken where the pages leave a step open:

* the residual is the difference between the decision scale's full attention
  output and its sparse one, R = O_full^D - O_sparse^D, per (b, h, query,
  head dim); the sparse output at D is block-sparse attention over the
  decision tiles' own selection (the CS4A lists mapped from D to D);
* the upsampling is nearest-neighbour on the token grid, with the same integer
  projection used everywhere else: target token (y, x) at side h_T takes the
  residual of token (floor(y h_D / h_T), floor(x h_D / h_T)) at side h_D;
* the correction adds it: O^T = O_sparse^T + up(R).
"""
from __future__ import annotations

import numpy as np


def residual(o_full: np.ndarray, o_sparse: np.ndarray) -> np.ndarray:
    """R = O_full - O_sparse at the decision scale, float64, [..., N_D, d]."""
    return np.asarray(o_full, dtype=np.float64) - np.asarray(o_sparse, dtype=np.float64)


def nearest_source(side_d: int, side_t: int) -> np.ndarray:
    """For every target token t = y * side_t + x (raster order), the index of
    the decision-scale token it reads: floor(y h_D/h_T) * h_D + floor(x h_D/h_T)."""
    y = np.arange(side_t)
    src = (y * side_d) // side_t
    return (src[:, None] * side_d + src[None, :]).reshape(-1)


def upsample(r: np.ndarray, side_d: int, side_t: int) -> np.ndarray:
    """Nearest-neighbour upsampling of [..., side_d^2, d] to [..., side_t^2, d]."""
    assert r.shape[-2] == side_d * side_d
    return r[..., nearest_source(side_d, side_t), :]


def correct(o_t: np.ndarray, o_full_d: np.ndarray, o_sparse_d: np.ndarray, side_d: int, side_t: int) -> np.ndarray:
    """O^T + up(O_full^D - O_sparse^D), float64."""
    return np.asarray(o_t, dtype=np.float64) + upsample(residual(o_full_d, o_sparse_d), side_d, side_t)

"""Seeded synthetic inputs for the multi-scale attention workloads.

This module only draws numbers: it holds none of the attention, masking,
scoring or mapping arithmetic.  Both the HIP path (through the Python
binding) and the CPU oracle are fed from here, so that the two sides see
bit-identical inputs.

Workload shapes follow the SparVAR pages (the last, high-resolution scales
of next-scale VAR generation, where one query scale attends to the
concatenated key/value cache of every earlier scale plus itself).  The pages
measured on real Infinity activations, which are not available; the value
recipe below stands in for them:

* ``gaussian``: Q, K, V ~ N(0, 1) (the small fp32 case).
* ``spatial``: per (batch, head) two random-Fourier fields F_K, F_V mapping
  the unit square to R^d, F(p) = sqrt(2) cos(Omega p + phi) with
  Omega ~ N(0, (2 pi / ell)^2), phi ~ U[0, 2 pi), ell = 0.25, sampled at the
  token centres ((x + 1/2) / h, (y + 1/2) / h) of every scale.
  K = F_K + 0.5 N(0,1), V = F_V + 0.5 N(0,1), Q = F_K(query scale) + 0.5 N(0,1),
  so attention is spatially local.  Keys of the sink scales get
  2 * mu added, mu being the unit mean of F_K over the largest grid (the mean
  query direction), which makes the early scales attention sinks.

Every stream is independent: numpy ``default_rng`` keyed by
(seed, workload id, b, h, role).  Values are rounded on the host to bfloat16
(round to nearest even) where the workload is bf16.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "SCHEDULE_13",
    "SCHEDULE_16",
    "TINY_SIDES",
    "bf16_bits",
    "bf16_bits_to_f32",
    "round_bf16",
    "gaussian_qkv",
    "SpatialField",
]

# Scale schedules (token-grid side of each scale, coarse to fine).
TINY_SIDES = (1, 2, 4, 8, 16)
SCHEDULE_13 = (1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64)
SCHEDULE_16 = SCHEDULE_13 + (80, 96, 128)

_ROLE = {"q": 1, "k": 2, "v": 3, "fk": 4, "fv": 5, "qn": 6, "kn": 7, "vn": 8}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    # NaN stays NaN (not produced by the generators, kept for completeness)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


def _rng(seed: int, wid: int, b: int, h: int, role: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(wid), int(b), int(h), _ROLE[role]])


def gaussian_qkv(seed: int, wid: int, B: int, H: int, nq: int, nk: int, d: int):
    """Q [B,H,nq,d], K and V [B,H,nk,d], all N(0,1), float32."""
    q = np.empty((B, H, nq, d), np.float32)
    k = np.empty((B, H, nk, d), np.float32)
    v = np.empty((B, H, nk, d), np.float32)
    for b in range(B):
        for h in range(H):
            q[b, h] = _rng(seed, wid, b, h, "q").standard_normal((nq, d), dtype=np.float32)
            k[b, h] = _rng(seed, wid, b, h, "k").standard_normal((nk, d), dtype=np.float32)
            v[b, h] = _rng(seed, wid, b, h, "v").standard_normal((nk, d), dtype=np.float32)
    return q, k, v


def _grid_centres(side: int) -> np.ndarray:
    """Token centres of a side x side grid in raster order, as (x, y) in [0,1)^2."""
    ys, xs = np.meshgrid(np.arange(side), np.arange(side), indexing="ij")
    return np.stack([(xs.ravel() + 0.5) / side, (ys.ravel() + 0.5) / side], axis=1)


class SpatialField:
    """Per-head smooth spatial fields; see the module docstring for the recipe."""

    ELL = 0.25

    def __init__(self, seed: int, wid: int, B: int, H: int, d: int):
        self.seed, self.wid, self.B, self.H, self.d = seed, wid, B, H, d
        self._params = {}
        for b in range(B):
            for h in range(H):
                for role in ("fk", "fv"):
                    g = _rng(seed, wid, b, h, role)
                    omega = g.normal(0.0, 2.0 * np.pi / self.ELL, size=(d, 2))
                    phi = g.uniform(0.0, 2.0 * np.pi, size=d)
                    self._params[(b, h, role)] = (omega, phi)

    def _field(self, b: int, h: int, role: str, side: int) -> np.ndarray:
        omega, phi = self._params[(b, h, role)]
        p = _grid_centres(side)
        return (np.sqrt(2.0) * np.cos(p @ omega.T + phi)).astype(np.float32)

    def _sink_dir(self, b: int, h: int, largest_side: int) -> np.ndarray:
        mu = self._field(b, h, "fk", largest_side).astype(np.float64).mean(axis=0)
        n = np.linalg.norm(mu)
        return (mu / n if n > 0 else np.zeros_like(mu)).astype(np.float32)

    def keys_values(self, sides, n_sink: int, largest_side: int | None = None):
        """K and V [B,H,Nk,d] float32 over the concatenated scales ``sides``."""
        sides = list(sides)
        largest_side = max(sides) if largest_side is None else largest_side
        nk = sum(s * s for s in sides)
        k = np.empty((self.B, self.H, nk, self.d), np.float32)
        v = np.empty((self.B, self.H, nk, self.d), np.float32)
        for b in range(self.B):
            for h in range(self.H):
                fk = np.concatenate([self._field(b, h, "fk", s) for s in sides])
                fv = np.concatenate([self._field(b, h, "fv", s) for s in sides])
                kn = _rng(self.seed, self.wid, b, h, "kn").standard_normal(fk.shape, dtype=np.float32)
                vn = _rng(self.seed, self.wid, b, h, "vn").standard_normal(fv.shape, dtype=np.float32)
                kk = fk + 0.5 * kn
                n_sink_tok = sum(s * s for s in sides[:n_sink])
                if n_sink_tok:
                    kk[:n_sink_tok] += 2.0 * self._sink_dir(b, h, largest_side)
                k[b, h] = kk
                v[b, h] = fv + 0.5 * vn
        return k, v

    def queries(self, side: int):
        """Q [B,H,side*side,d] float32 at a scale of the given side."""
        q = np.empty((self.B, self.H, side * side, self.d), np.float32)
        for b in range(self.B):
            for h in range(self.H):
                f = self._field(b, h, "fk", side)
                # a separate stream per query side, so each scale's noise is independent
                g = np.random.default_rng([int(self.seed), int(self.wid), b, h, _ROLE["qn"], int(side)])
                q[b, h] = f + 0.5 * g.standard_normal(f.shape, dtype=np.float32)
        return q

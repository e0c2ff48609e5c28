"""Multi-scale token grid and its 2-D tiles (oracle; test infrastructure).

The pages (SparVAR, ai.info summary, "What This Paper Is About") describe
next-scale generation: scale k's tokens attend to the tokens of every earlier
scale and of scale k itself.  Here the key/value cache of a query scale q is
the concatenation of scales 0..q, each scale a side x side grid in raster
(row-major) order.

The block mask the pages derive from the token mask (ai.info, "Methodology in
Plain English") is read here with blocks as square t x t tiles of one scale's
grid; tiles on the right/bottom edge of a grid whose side is not a multiple of
t are partial.  Key tiles are numbered scale by scale, raster order within a
scale; query tiles are numbered in raster order over the query scale.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def scale_offsets(sides) -> list[int]:
    """Token offset of every scale in the concatenated cache (length S + 1)."""
    off = [0]
    for s in sides:
        off.append(off[-1] + int(s) * int(s))
    return off


def tiles_per_side(side: int, t: int) -> int:
    return -(-int(side) // int(t))


@dataclass(frozen=True)
class Tile:
    scale: int
    a: int  # tile row within the scale
    b: int  # tile column within the scale
    row0: int
    col0: int
    rows: int
    cols: int
    side: int
    offset: int  # token offset of the scale

    def tokens(self) -> np.ndarray:
        """Token indices of the tile in the concatenated cache, raster order."""
        r = np.arange(self.row0, self.row0 + self.rows)
        c = np.arange(self.col0, self.col0 + self.cols)
        return (self.offset + r[:, None] * self.side + c[None, :]).ravel()


def key_tiles(sides, q_scale: int, t: int) -> list[Tile]:
    """All tiles of scales 0..q_scale, in key-tile id order."""
    off = scale_offsets(sides)
    out = []
    for s in range(q_scale + 1):
        h = int(sides[s])
        nb = tiles_per_side(h, t)
        for a in range(nb):
            for b in range(nb):
                r0, c0 = a * t, b * t
                out.append(Tile(s, a, b, r0, c0, min(t, h - r0), min(t, h - c0), h, off[s]))
    return out


def query_tiles(sides, q_scale: int, t: int) -> list[Tile]:
    """Tiles of the query scale; token indices are local to the query scale."""
    h = int(sides[q_scale])
    nb = tiles_per_side(h, t)
    return [Tile(q_scale, a, b, a * t, b * t, min(t, h - a * t), min(t, h - b * t), h, 0)
            for a in range(nb) for b in range(nb)]


def key_token_coords(sides, q_scale: int):
    """(scale, y, x) of every key token of scales 0..q_scale, cache order."""
    sc, ys, xs = [], [], []
    for s in range(q_scale + 1):
        h = int(sides[s])
        y, x = np.meshgrid(np.arange(h), np.arange(h), indexing="ij")
        sc.append(np.full(h * h, s))
        ys.append(y.ravel())
        xs.append(x.ravel())
    return np.concatenate(sc), np.concatenate(ys), np.concatenate(xs)


def key_token_tile(sides, q_scale: int, t: int) -> np.ndarray:
    """Key-tile id of every key token."""
    ids = np.empty(scale_offsets(sides)[q_scale + 1], np.int64)
    for i, tile in enumerate(key_tiles(sides, q_scale, t)):
        ids[tile.tokens()] = i
    return ids


def counts(sides, q_scale: int, t: int):
    """(nqb, nkb, nq, nk) for a query scale."""
    h = int(sides[q_scale])
    nqb = tiles_per_side(h, t) ** 2
    nkb = sum(tiles_per_side(sides[s], t) ** 2 for s in range(q_scale + 1))
    return nqb, nkb, h * h, scale_offsets(sides)[q_scale + 1]

"""CSLA block mask (oracle; test infrastructure).

Source: SparVAR, ai.info summary, "Methodology in Plain English" (the second
module, CSLA) and "Main Findings" (the sink ablation: sink = scales <= 5,
window sizes 3/5/7).  What the module computes, in this implementation's
terms: the position of a query of a late scale is carried onto every coarser
grid; on each of those grids only the keys close to that position survive;
every key of the first few ("sink") scales survives for every query; and
the surviving token pairs decide which (query block, key block) pairs are
computed.

Readings taken where the pages leave a step open:

* projection: integer nearest-neighbour, (y, x) at side H -> (floor(y h / H),
  floor(x h / H)) at side h;
* window: square (Chebyshev) of radius r_s tokens of the key scale's grid,
  i.e. side 2 r_s + 1; r_s < 0 drops the scale (sinks excepted); the query
  scale itself is windowed too (its projection is the identity);
* sink: the first n_sink scales (0-based s < n_sink) are kept whole;
* blocks: a (query tile, key tile) pair is kept iff any of its token pairs is
  kept (the step that turns the token mask into a block mask).

Budget variant (used to sweep block sparsity at fixed cost): per query tile,
key tiles are ranked by (not sink, admission radius, -scale, id) and the
first max(k, number of sink tiles + 1) are kept, the admission radius of a
pair being the smallest window radius at which the token rule keeps it.
"""
from __future__ import annotations

import numpy as np

from . import geometry as G


def token_mask_for_query_tile(sides, q_scale: int, t: int, n_sink: int, radius, qtile: G.Tile) -> np.ndarray:
    """bool [queries of the tile, Nk]: the token-level CSLA keep rule."""
    H = int(sides[q_scale])
    ks, ky, kx = G.key_token_coords(sides, q_scale)
    h_of_key = np.asarray(sides, np.int64)[ks]
    r_of_key = np.asarray([radius[s] for s in range(q_scale + 1)], np.int64)[ks]
    rows = []
    for yy in range(qtile.row0, qtile.row0 + qtile.rows):
        for xx in range(qtile.col0, qtile.col0 + qtile.cols):
            py = (yy * h_of_key) // H          # projection of the query onto each key's scale
            px = (xx * h_of_key) // H
            in_window = (np.abs(ky - py) <= r_of_key) & (np.abs(kx - px) <= r_of_key) & (r_of_key >= 0)
            rows.append((ks < n_sink) | in_window)
    return np.stack(rows)


def _any_per_tile(token_rows: np.ndarray, tile_of_key: np.ndarray, nkb: int) -> np.ndarray:
    hit = token_rows.any(axis=0)
    out = np.zeros(nkb, bool)
    out[np.unique(tile_of_key[hit])] = True
    return out


def block_mask(sides, q_scale: int, t: int, n_sink: int, radius) -> np.ndarray:
    """bool [nqb, nkb]: kept (query tile, key tile) pairs of the CSLA mask."""
    tiles = G.key_tiles(sides, q_scale, t)
    tile_of_key = G.key_token_tile(sides, q_scale, t)
    qts = G.query_tiles(sides, q_scale, t)
    out = np.zeros((len(qts), len(tiles)), bool)
    for i, qt in enumerate(qts):
        out[i] = _any_per_tile(token_mask_for_query_tile(sides, q_scale, t, n_sink, radius, qt),
                               tile_of_key, len(tiles))
    return out


def admission_radius(sides, q_scale: int, t: int) -> np.ndarray:
    """int [nqb, nkb]: min over token pairs of the Chebyshev distance between
    the key token and the query token's projection onto the key's scale."""
    H = int(sides[q_scale])
    ks, ky, kx = G.key_token_coords(sides, q_scale)
    h_of_key = np.asarray(sides, np.int64)[ks]
    tiles = G.key_tiles(sides, q_scale, t)
    tile_of_key = G.key_token_tile(sides, q_scale, t)
    qts = G.query_tiles(sides, q_scale, t)
    out = np.zeros((len(qts), len(tiles)), np.int64)
    for i, qt in enumerate(qts):
        best = np.full(ks.shape, np.iinfo(np.int64).max)
        for yy in range(qt.row0, qt.row0 + qt.rows):
            for xx in range(qt.col0, qt.col0 + qt.cols):
                dy = np.abs(ky - (yy * h_of_key) // H)
                dx = np.abs(kx - (xx * h_of_key) // H)
                best = np.minimum(best, np.maximum(dy, dx))
        per_tile = np.full(len(tiles), np.iinfo(np.int64).max)
        np.minimum.at(per_tile, tile_of_key, best)
        out[i] = per_tile
    return out


def budget_mask(sides, q_scale: int, t: int, n_sink: int, budget: int) -> np.ndarray:
    """bool [nqb, nkb]: per query tile keep the first max(budget, sink tiles + 1)
    key tiles in (not sink, admission radius, -scale, id) order."""
    tiles = G.key_tiles(sides, q_scale, t)
    dist = admission_radius(sides, q_scale, t)
    is_sink = np.array([tl.scale < n_sink for tl in tiles])
    scale = np.array([tl.scale for tl in tiles])
    keep_n = min(len(tiles), max(int(budget), int(is_sink.sum()) + 1))
    out = np.zeros(dist.shape, bool)
    for i in range(dist.shape[0]):
        order = sorted(range(len(tiles)), key=lambda j: (not is_sink[j], dist[i, j], -scale[j], j))
        out[i, order[:keep_n]] = True
    return out


def lists_from_mask(mask: np.ndarray):
    """Ascending kept key-tile ids per row: (cnt int32 [rows], idx int32 [rows, nkb], -1 padded)."""
    rows, nkb = mask.shape[-2], mask.shape[-1]
    flat = mask.reshape(-1, nkb)
    cnt = flat.sum(axis=1).astype(np.int32)
    idx = np.full(flat.shape, -1, np.int32)
    for r in range(flat.shape[0]):
        nz = np.flatnonzero(flat[r])
        idx[r, : nz.size] = nz
    return cnt.reshape(mask.shape[:-1]), idx.reshape(mask.shape)


def sparsity(mask: np.ndarray, sides, q_scale: int, t: int):
    """(count sparsity, token-weighted sparsity) of a [.., nqb, nkb] block mask."""
    qsz = np.array([tl.rows * tl.cols for tl in G.query_tiles(sides, q_scale, t)], np.float64)
    ksz = np.array([tl.rows * tl.cols for tl in G.key_tiles(sides, q_scale, t)], np.float64)
    m = mask.reshape(-1, *mask.shape[-2:]).astype(np.float64)
    count = 1.0 - m.mean()
    pairs = np.einsum("i,nij,j->", qsz, m, ksz) / m.shape[0]
    return count, 1.0 - pairs / (qsz.sum() * ksz.sum())

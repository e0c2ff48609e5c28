"""CS4A: decision-scale block scores, top-p selection, cross-scale index mapping
(oracle; test infrastructure).

Source: SparVAR, ai.info summary, "Methodology in Plain English" (the first
module, CS4A) and "Main Findings" (decision scale fixed to a mid scale, scale
10); gptget.net summary, "Abstract" (dynamic prediction of later scales'
sparse pattern from a sparse decision scale through index mapping).  Full
attention is computed at the decision scale D, the attention map is split into
query blocks, weights are summed within each (query block, key block), the key
blocks that matter most are selected, and their indices are rescaled to the
later scales, optionally with the sink region concatenated.

Readings taken where the pages leave a step open:

* score[Q, K] = (1/|Q|) sum_{q in Q, k in K} P[q, k], P the softmax of
  Q_D K_{<=D}^T / sqrt(d) over all keys of scales 0..D, so each query tile's
  row of scores sums to 1 (the pages add the weights up per block; the
  constant factor does not change any ranking);
* selection keeps the most massive key tiles up to a cumulative mass top_p
  (the crossing tile included); the alternative Top-K rule (the pages give a
  Top-K ratio of about 0.2 as the stable setting, "Main Findings", decision
  scale item) keeps the first ceil(frac * nkb) tiles of the same order.  Scores are first quantised to integers
  m = floor(score * 2^24) from their float32 value, tiles are ordered by
  (m descending, id ascending), the threshold is ceil(top_p * sum m) computed
  in IEEE double, and the shortest prefix whose sum reaches it is kept;
* index mapping for target scale T: target query tile (i, j) takes the
  selection of its parent tile (floor(i nb_D / nb_T), floor(j nb_D / nb_T))
  at D; selected tiles of scales below D are kept as they are (the same
  tokens); a selected tile of scale D is replaced, on every scale s with
  D <= s <= T, by the key tiles that hold a token whose cell overlaps the
  selected tile's region of the unit square; the sink tiles are added.
"""
from __future__ import annotations

import math

import numpy as np

from . import geometry as G

QUANT_SCALE = float(2 ** 24)


def block_scores(q_d: np.ndarray, k: np.ndarray, sides, d_scale: int, t: int, softmax_scale: float) -> np.ndarray:
    """float64 [B, H, nqb_D, nkb_D].  q_d [B,H,N_D,d], k [B,H,>=Nk_D,d]."""
    qts = G.query_tiles(sides, d_scale, t)
    kts = G.key_tiles(sides, d_scale, t)
    nk = G.scale_offsets(sides)[d_scale + 1]
    B, Hh = q_d.shape[:2]
    out = np.zeros((B, Hh, len(qts), len(kts)))
    for b in range(B):
        for h in range(Hh):
            s = q_d[b, h].astype(np.float64) @ k[b, h, :nk].astype(np.float64).T * softmax_scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            for i, qt in enumerate(qts):
                qtok = qt.tokens()
                rows = p[qtok]
                for j, kt in enumerate(kts):
                    out[b, h, i, j] = rows[:, kt.tokens()].sum() / qtok.size
    return out


def quantise(scores_f32: np.ndarray) -> np.ndarray:
    """int64 floor(score * 2^24) of float32 scores (exact: a power-of-two scaling)."""
    s = np.asarray(scores_f32, np.float32).astype(np.float64)
    return np.floor(s * QUANT_SCALE).astype(np.int64)


def top_p_row(scores_row_f32: np.ndarray, top_p: float) -> np.ndarray:
    """Ascending ids of the tiles kept for one query tile."""
    m = quantise(scores_row_f32)
    order = sorted(range(m.size), key=lambda j: (-int(m[j]), j))
    total = int(m.sum())
    threshold = math.ceil(float(np.float32(top_p)) * float(total))
    kept, acc = [], 0
    for j in order:
        if acc >= threshold:
            break
        kept.append(j)
        acc += int(m[j])
    return np.array(sorted(kept), np.int64)


def top_p_select(scores_f32: np.ndarray, top_p: float):
    """(cnt int32 [..., nqb], idx int32 [..., nqb, nkb] ascending, -1 padded)."""
    sc = np.asarray(scores_f32, np.float32)
    flat = sc.reshape(-1, sc.shape[-1])
    cnt = np.zeros(flat.shape[0], np.int32)
    idx = np.full(flat.shape, -1, np.int32)
    for r in range(flat.shape[0]):
        kept = top_p_row(flat[r], top_p)
        cnt[r] = kept.size
        idx[r, : kept.size] = kept
    return cnt.reshape(sc.shape[:-1]), idx.reshape(sc.shape)


def top_k_count(nkb: int, frac: float) -> int:
    """Tiles kept per query tile by the Top-K-fraction rule: ceil of the
    float32 product frac * nkb (so that 0.2 of 160 is 32, not 33 as the
    float32 value of 0.2, slightly above 0.2, would give in double), clamped
    to [1, nkb]."""
    k = math.ceil(float(np.float32(frac) * np.float32(nkb)))
    return min(max(k, 1), nkb)


def top_k_row(scores_row_f32: np.ndarray, frac: float) -> np.ndarray:
    """Ascending ids of the top_k_count tiles first in the (m descending, id
    ascending) order of the quantised scores."""
    m = quantise(scores_row_f32)
    order = sorted(range(m.size), key=lambda j: (-int(m[j]), j))
    return np.array(sorted(order[: top_k_count(m.size, frac)]), np.int64)


def top_k_select(scores_f32: np.ndarray, frac: float):
    """(cnt int32 [..., nqb], idx int32 [..., nqb, nkb] ascending, -1 padded)."""
    sc = np.asarray(scores_f32, np.float32)
    flat = sc.reshape(-1, sc.shape[-1])
    cnt = np.zeros(flat.shape[0], np.int32)
    idx = np.full(flat.shape, -1, np.int32)
    for r in range(flat.shape[0]):
        kept = top_k_row(flat[r], frac)
        cnt[r] = kept.size
        idx[r, : kept.size] = kept
    return cnt.reshape(sc.shape[:-1]), idx.reshape(sc.shape)


def _footprint_tiles(sides, t: int, d_scale: int, sel_tile: G.Tile, s: int) -> list[int]:
    """Key-tile ids (scale s, ids of the T geometry) holding a token whose cell
    overlaps the region of the unit square covered by ``sel_tile`` (scale D)."""
    hD, hs = int(sides[d_scale]), int(sides[s])
    y0, y1 = sel_tile.row0, sel_tile.row0 + sel_tile.rows      # rows [y0, y1) of scale D
    x0, x1 = sel_tile.col0, sel_tile.col0 + sel_tile.cols
    # token y' of scale s covers [y'/hs, (y'+1)/hs); overlap with [y0/hD, y1/hD) iff
    # y' * hD < y1 * hs and (y' + 1) * hD > y0 * hs (exact in integers)
    ys = [y for y in range(hs) if y * hD < y1 * hs and (y + 1) * hD > y0 * hs]
    xs = [x for x in range(hs) if x * hD < x1 * hs and (x + 1) * hD > x0 * hs]
    nb = G.tiles_per_side(hs, t)
    base = sum(G.tiles_per_side(sides[u], t) ** 2 for u in range(s))
    return sorted({base + (y // t) * nb + (x // t) for y in ys for x in xs})


def map_indices(sel_cnt: np.ndarray, sel_idx: np.ndarray, sides, d_scale: int, t_scale: int, t: int,
                n_sink: int):
    """Map decision-scale selections [..., nqb_D] to target-scale lists
    (cnt int32 [..., nqb_T], idx int32 [..., nqb_T, nkb_T] ascending, -1 padded)."""
    ktD = G.key_tiles(sides, d_scale, t)
    ktT = G.key_tiles(sides, t_scale, t)
    nbD = G.tiles_per_side(sides[d_scale], t)
    nbT = G.tiles_per_side(sides[t_scale], t)
    sinks = [j for j, tl in enumerate(ktT) if tl.scale < n_sink]
    lead = sel_cnt.shape[:-1]
    cnt_flat = sel_cnt.reshape(-1, sel_cnt.shape[-1])
    idx_flat = sel_idx.reshape(-1, *sel_idx.shape[-2:])
    out_cnt = np.zeros((cnt_flat.shape[0], nbT * nbT), np.int32)
    out_idx = np.full((cnt_flat.shape[0], nbT * nbT, len(ktT)), -1, np.int32)
    for r in range(cnt_flat.shape[0]):
        for ti in range(nbT):
            for tj in range(nbT):
                parent = (ti * nbD // nbT) * nbD + (tj * nbD // nbT)
                kept = set(sinks)
                for j in idx_flat[r, parent, : cnt_flat[r, parent]]:
                    tl = ktD[int(j)]
                    if tl.scale < d_scale:
                        kept.add(int(j))          # same tile id in the target geometry
                    else:
                        for s in range(d_scale, t_scale + 1):
                            kept.update(_footprint_tiles(sides, t, d_scale, tl, s))
                ids = sorted(kept)
                q = ti * nbT + tj
                out_cnt[r, q] = len(ids)
                out_idx[r, q, : len(ids)] = ids
    return out_cnt.reshape(*lead, nbT * nbT), out_idx.reshape(*lead, nbT * nbT, len(ktT))

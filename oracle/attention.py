"""Masked softmax attention (oracle; test infrastructure).

Source: SparVAR, ai.info summary, "Main Findings" (block-wise sparse kernel
vs dense FlashAttention on the last scale) and "Methodology in Plain English"
(the block mask decides which keys a query attends to).  The sparse kernel
computes ordinary scaled-dot-product attention restricted to the keys of the
kept blocks, so the oracle applies the block mask token-wise as -inf to dense
softmax attention:

    S = Q K^T * softmax_scale,  S[q, k] = -inf where (tile(q), tile(k)) is not kept,
    O = softmax(S) V,  lse[q] = log sum_k exp(S[q, k])   (natural log).

All arithmetic is float64 on the values given (the bf16-rounded inputs upcast).
A query with no kept key gets O = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

from . import geometry as G


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray, softmax_scale: float):
    """q [nq,d], k/v [nk,d], keep bool [nq,nk] -> (O float64 [nq,d], lse float64 [nq])."""
    s = q.astype(np.float64) @ k.astype(np.float64).T * softmax_scale
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v.astype(np.float64)) / np.where(l > 0, l, 1.0)
    lse = (m + np.log(np.where(l > 0, l, 1.0)))[:, 0]
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def tile_token_mask(kept_tiles, sides, q_scale: int, t: int) -> np.ndarray:
    """bool [Nk]: the key tokens covered by a set of kept key-tile ids."""
    tiles = G.key_tiles(sides, q_scale, t)
    keep = np.zeros(G.scale_offsets(sides)[q_scale + 1], bool)
    for j in kept_tiles:
        keep[tiles[int(j)].tokens()] = True
    return keep


def block_sparse_attention(q, k, v, sides, q_scale: int, t: int, kv_cnt, kv_idx, softmax_scale: float,
                           q_tiles=None, bh=None):
    """Block-sparse attention of one query scale over the multi-scale cache.

    q [B,H,Nq,d] (query-scale tokens, raster order), k/v [B,H,Nk,d].
    kv_cnt [nqb] / kv_idx [nqb,nkb] shared by every (b,h), or kv_cnt [B,H,nqb] /
    kv_idx [B,H,nqb,nkb] per (b,h).  ``q_tiles`` restricts the query tiles
    computed, ``bh`` the (b,h) pairs; rows not computed are left NaN.
    Returns (O float64 [B,H,Nq,d], lse float64 [B,H,Nq]).
    """
    B, Hh, nq, d = q.shape
    qts = G.query_tiles(sides, q_scale, t)
    o = np.full((B, Hh, nq, d), np.nan)
    lse = np.full((B, Hh, nq), np.nan)
    kv_cnt = np.asarray(kv_cnt)
    kv_idx = np.asarray(kv_idx)
    pairs = bh if bh is not None else [(b, h) for b in range(B) for h in range(Hh)]
    sel = range(len(qts)) if q_tiles is None else q_tiles
    for (b, h) in pairs:
        cnt = kv_cnt if kv_cnt.ndim == 1 else kv_cnt[b, h]
        idx = kv_idx if kv_idx.ndim == 2 else kv_idx[b, h]
        for i in sel:
            qtok = qts[i].tokens()
            keep_row = tile_token_mask(idx[i, : cnt[i]], sides, q_scale, t)
            keep = np.broadcast_to(keep_row, (qtok.size, keep_row.size))
            oi, li = softmax_attention(q[b, h, qtok], k[b, h, : keep_row.size], v[b, h, : keep_row.size],
                                       keep, softmax_scale)
            o[b, h, qtok] = oi
            lse[b, h, qtok] = li
    return o, lse


def dense_attention(q, k, v, softmax_scale: float, q_rows=None, bh=None):
    """Dense attention, q [B,H,nq,d], k/v [B,H,nk,d]; optional query-row subset."""
    B, Hh, nq, d = q.shape
    rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    o = np.full((B, Hh, nq, d), np.nan)
    lse = np.full((B, Hh, nq), np.nan)
    pairs = bh if bh is not None else [(b, h) for b in range(B) for h in range(Hh)]
    for (b, h) in pairs:
        keep = np.ones((rows.size, k.shape[2]), bool)
        oi, li = softmax_attention(q[b, h, rows], k[b, h], v[b, h], keep, softmax_scale)
        o[b, h, rows] = oi
        lse[b, h, rows] = li
    return o, lse


def token_masked_attention(q, k, v, sides, q_scale: int, t: int, n_sink: int, radius, softmax_scale: float,
                           q_tiles=None, bh=None):
    """Attention under the token-level CSLA mask itself (SparVAR, ai.info
    summary, "Key Contributions" item 3: the naive token-wise sparse attention
    baseline the block kernel is compared with; "Methodology in Plain
    English", second module: a key is kept iff its scale is a sink or it lies
    in the per-scale window around the query's projection).  The same result
    as block-sparse attention over the CSLA tiles with the token rule applied
    inside them (every kept token pair lies in a kept tile).  q [B,H,side^2,d],
    k/v [B,H,Nk,d]; optional query-tile / (b, h) subsets; other rows NaN."""
    from . import csla
    B, Hh, nq, d = q.shape
    qts = G.query_tiles(sides, q_scale, t)
    sel = range(len(qts)) if q_tiles is None else q_tiles
    o = np.full((B, Hh, nq, d), np.nan)
    lse = np.full((B, Hh, nq), np.nan)
    pairs = bh if bh is not None else [(b, h) for b in range(B) for h in range(Hh)]
    for r in sel:
        qt = qts[r]
        rows = qt.tokens()
        keep = csla.token_mask_for_query_tile(sides, q_scale, t, n_sink, radius, qt)
        for (b, h) in pairs:
            oi, li = softmax_attention(q[b, h, rows], k[b, h], v[b, h], keep, softmax_scale)
            o[b, h, rows] = oi
            lse[b, h, rows] = li
    return o, lse

"""The per-scale loop with both sparse modules (oracle; test infrastructure).

Source: SparVAR, ai.info summary, "Main Findings" (the decision scale is
fixed to a mid-scale of the schedule; the two modules are added one after
the other, CS4A first, then the O_cache correction, then CSLA; the default
CSLA configuration keeps the scales up to the fifth as sinks and uses window
sizes 3, 5 and 7 for the last three scales) and "Methodology in Plain
English" (CS4A: full attention at the decision scale, block scores,
selection, mapping to the later scales, the residual upsampled onto their
sparse outputs; CSLA: a mask built from the sink and the cross-scale window,
independent of the decision scale).

Readings taken where the pages leave a step open:

* plan of one generation step, query scale by query scale (0-based q, D the
  decision scale): q < D attends densely; q = D attends densely (the full
  attention the scoring needs) and also block-sparsely over its own
  selection (the sparse output whose difference to the full one is the
  residual); every q > D attends block-sparsely over its CS4A-mapped tiles,
  joined with its CSLA tiles when q is one of the last len(windows) scales,
  and its output gets the O_cache correction;
* window schedule: the i-th of the last len(windows) query scales uses the
  odd window windows[i] on every key scale it attends to, i.e. the radius
  (windows[i] - 1) / 2 in tokens of each key scale's grid;
* join: the union of the two kept-tile sets (adding a module adds the pairs
  it keeps); the intersection is kept as the alternative reading.  The pages'
  speed figures do not decide between the two.
"""
from __future__ import annotations

import numpy as np

from . import attention as A
from . import cs4a as C
from . import csla as L
from . import geometry as G
from . import ocache as OC

JOINS = ("union", "intersection")


def window_radius(n_scales: int, q_scale: int, windows=(3, 5, 7)):
    """Per-key-scale radii [q_scale + 1] of a query scale under the window
    schedule of the last len(windows) scales."""
    first = n_scales - len(windows)
    if not first <= q_scale < n_scales:
        raise ValueError("query scale outside the windowed scales")
    w = int(windows[q_scale - first])
    if w < 1 or w % 2 == 0:
        raise ValueError("windows are odd and >= 1")
    return [(w - 1) // 2] * (q_scale + 1)


def plan(n_scales: int, d_scale: int, n_windows: int):
    """Per query scale: "dense", "decision", "cs4a" or "cs4a+csla"."""
    out = []
    for q in range(n_scales):
        if q < d_scale:
            out.append("dense")
        elif q == d_scale:
            out.append("decision")
        else:
            out.append("cs4a+csla" if q >= n_scales - n_windows else "cs4a")
    return out


def join_masks(a: np.ndarray, b: np.ndarray, join: str) -> np.ndarray:
    """Element-wise union or intersection of two block masks (b broadcasts)."""
    if join == "union":
        return np.logical_or(a, b)
    if join == "intersection":
        return np.logical_and(a, b)
    raise ValueError(join)


def mask_from_lists(cnt: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """bool [..., rows, nkb] from ascending lists (cnt [..., rows], idx [..., rows, nkb])."""
    nkb = idx.shape[-1]
    c = cnt.reshape(-1)
    ii = idx.reshape(-1, nkb)
    m = np.zeros((c.size, nkb), bool)
    for r in range(c.size):
        m[r, ii[r, : c[r]]] = True
    return m.reshape(idx.shape)


def scale_loop(queries, k, v, sides, t: int, d_scale: int, n_sink: int, top_p: float, windows, softmax_scale: float,
               join: str = "union", radius_override=None):
    """One generation step of attention over every query scale.

    queries[q] [B,H,side_q^2,d] per query scale, k/v [B,H,Nk,d] over all
    scales (each query scale reads its prefix).  Returns a dict per query scale
    with "o" (float64 [B,H,N_q,d]) and, for the sparse scales, "cnt"/"idx"
    (the kept lists attended).  Scores and selection follow the CS4A oracle:
    float32 block scores (the precision the selection rule is stated in).
    ``radius_override`` replaces the window schedule's radii on every joined
    scale (a list of per-key-scale radii long enough for the last scale).
    """
    n = len(sides)
    steps = plan(n, d_scale, len(windows))
    off = G.scale_offsets(sides)
    out = {}
    o_full_d = o_sparse_d = None
    for q, kind in enumerate(steps):
        nk = off[q + 1]
        kq, vq = k[:, :, :nk], v[:, :, :nk]
        if kind == "dense":
            out[q] = {"o": A.dense_attention(queries[q], kq, vq, softmax_scale)[0]}
            continue
        if kind == "decision":
            o_full_d = A.dense_attention(queries[q], kq, vq, softmax_scale)[0]
            scores = C.block_scores(queries[q], kq, sides, d_scale, t, softmax_scale).astype(np.float32)
            sel_cnt, sel_idx = C.top_p_select(scores, top_p)
            cnt_d, idx_d = C.map_indices(sel_cnt, sel_idx, sides, d_scale, d_scale, t, n_sink)
            o_sparse_d = A.block_sparse_attention(queries[q], kq, vq, sides, q, t, cnt_d, idx_d, softmax_scale)[0]
            out[q] = {"o": o_full_d, "cnt": cnt_d, "idx": idx_d}
            continue
        cnt, idx = C.map_indices(sel_cnt, sel_idx, sides, d_scale, q, t, n_sink)
        if kind == "cs4a+csla":
            radius = window_radius(n, q, windows) if radius_override is None else list(radius_override)[: q + 1]
            csla = L.block_mask(sides, q, t, n_sink, radius)
            cnt, idx = L.lists_from_mask(join_masks(mask_from_lists(cnt, idx), csla, join))
        o_t = A.block_sparse_attention(queries[q], kq, vq, sides, q, t, cnt, idx, softmax_scale)[0]
        out[q] = {"o": OC.correct(o_t, o_full_d, o_sparse_d, sides[d_scale], sides[q]), "cnt": cnt, "idx": idx}
    return out

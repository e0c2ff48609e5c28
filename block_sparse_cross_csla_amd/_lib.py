"""ctypes binding of libvarsparse (include/varsparse.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory (outputs are
allocated here with torch.empty) and the current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvarsparse.so")
MAX_SCALES = 32
MAX_ATTN_TARGETS = 3
MAX_DENSE_TARGETS = 16
BF16, FP32 = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3

EXPORTS = (
    "varsparse_geom_counts",
    "varsparse_window_radius",
    "varsparse_build_mask",
    "varsparse_map_indices",
    "varsparse_map_indices_topk",
    "varsparse_map_indices_multi",
    "varsparse_attn_fwd",
    "varsparse_attn_fwd_token",
    "varsparse_attn_fwd_pair",
    "varsparse_attn_fwd_ocache",
    "varsparse_attn_fwd_multi",
    "varsparse_dense_attn_fwd",
    "varsparse_dense_attn_fwd_multi",
    "varsparse_ocache_correct",
    "varsparse_join_lists",
    "varsparse_strerror",
    "varsparse_last_hip_error",
)


class Geom(ctypes.Structure):
    _fields_ = [("n_scales", ctypes.c_int32), ("side", ctypes.c_int32 * MAX_SCALES), ("tile", ctypes.c_int32)]


class VarsparseError(RuntimeError):
    def __init__(self, code: int, where: str, hip: int = 0):
        self.code = code
        msg = f"{where}: {_LIB.varsparse_strerror(code).decode()} ({code})"
        if code == EHIP:
            msg += f", hipError {hip}"
        super().__init__(msg)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_sparse_cross_csla_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    PI32, PI64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    PG = ctypes.POINTER(Geom)
    lib.varsparse_geom_counts.argtypes = [PG, I32, PI32, PI32, PI64, PI64]
    lib.varsparse_window_radius.argtypes = [I32, I32, PI32, I32, PI32]
    lib.varsparse_build_mask.argtypes = [PG, I32, I32, PI32, I32, P, P, P, P]
    lib.varsparse_map_indices.argtypes = [PG, I32, I32, I32, F32, I32, I32, I32, I32,
                                          P, PI64, P, PI64, F32, P, P, P, P, P, P]
    lib.varsparse_map_indices_topk.argtypes = lib.varsparse_map_indices.argtypes
    lib.varsparse_attn_fwd.argtypes = [PG, I32, I32, I32, I32, I32, P, P, P, P, P, PI64, F32, P, P, I32, P]
    lib.varsparse_attn_fwd_token.argtypes = [PG, I32, I32, PI32, I32, I32, I32, P, P, P, P, P, PI64, F32, P, P, I32, P]
    lib.varsparse_map_indices_multi.argtypes = [PG, I32, I32, PI32, I32, I32, F32, I32, I32, I32, I32,
                                                P, PI64, P, PI64, F32, P, P, P, P]
    lib.varsparse_attn_fwd_pair.argtypes = [PG, I32, I32, I32, I32, P, P, P, P, P, PI64, F32, P, P, I32, P]
    lib.varsparse_dense_attn_fwd.argtypes = [I32, I32, I32, I32, I64, I64, P, P, P, P, P, PI64, F32, P]
    lib.varsparse_ocache_correct.argtypes = [I32, I32, I32, I32, I32, P, P, P, PI64, P]
    lib.varsparse_join_lists.argtypes = [I32, I32, I32, I32, P, P, I32, P, P, I32, P, P, P]
    lib.varsparse_strerror.argtypes = [ctypes.c_int]
    lib.varsparse_strerror.restype = ctypes.c_char_p
    lib.varsparse_last_hip_error.argtypes = []
    lib.varsparse_attn_fwd_ocache.argtypes = [PG, I32, I32, I32, I32, I32, P, P, P, P, P, PI64, F32, P, P, I32,
                                              P, P, PI64, P]
    lib.varsparse_attn_fwd_multi.argtypes = [PG, I32, PI32, I32, I32, I32, P, P, P, P, P, PI64, F32, P, P, I32,
                                             I32, P, P, PI64, P]
    lib.varsparse_dense_attn_fwd_multi.argtypes = [I32, I32, I32, I32, PI64, PI64, P, P, P, P, P, PI64, F32, P]
    for name in EXPORTS[:15]:
        getattr(lib, name).restype = ctypes.c_int
    lib.varsparse_last_hip_error.restype = ctypes.c_int
    return lib


_LIB = _load()


def lib():
    return _LIB


def _check(rc: int, where: str):
    if rc != OK:
        raise VarsparseError(rc, where, _LIB.varsparse_last_hip_error() if rc == EHIP else 0)


def make_geom(sides, tile: int) -> Geom:
    g = Geom()
    g.n_scales = len(sides)
    for i, s in enumerate(sides):
        g.side[i] = int(s)
    g.tile = int(tile)
    return g


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(*tensors):
    vals = []
    for t in tensors:
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
        vals.extend(t.stride()[:3])
    return (ctypes.c_int64 * len(vals))(*vals)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(cond, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_qkvo(q, k, v, out, lse, nq_expect: int, nk_min: int, bf16_only: bool):
    """Host-side checks that keep every kernel access inside the tensors: the
    library sees only pointers and strides."""
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v are [B, H, tokens, head_dim]")
    B, H, nq, d = q.shape
    _need(nq == nq_expect, f"q holds {nq} tokens per head, the query scale has {nq_expect}")
    for name, t in (("k", k), ("v", v)):
        _need(t.shape[0] == B and t.shape[1] == H and t.shape[3] == d, f"{name} {tuple(t.shape)} does not match q")
        _need(t.shape[2] >= nk_min, f"{name} holds {t.shape[2]} tokens, the attended cache needs {nk_min}")
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _need(len({q.dtype, k.dtype, v.dtype, out.dtype}) == 1, "q, k, v and out must share one dtype")
    if bf16_only:
        _need(q.dtype == torch.bfloat16, "this entry point takes bfloat16 tensors")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and lse.numel() == B * H * nq,
              "lse is a contiguous float32 [B, H, nq] tensor")


def _check_lists(kv_cnt, kv_idx, B: int, H: int, nqb: int, nkb: int):
    _need(kv_cnt.dtype == torch.int32 and kv_idx.dtype == torch.int32, "lists are int32")
    _need(kv_cnt.is_contiguous() and kv_idx.is_contiguous(), "lists must be contiguous")
    if kv_cnt.dim() == 1:
        _need(tuple(kv_cnt.shape) == (nqb,) and tuple(kv_idx.shape) == (nqb, nkb),
              f"shared lists are kv_cnt [{nqb}] and kv_idx [{nqb}, {nkb}]")
    else:
        _need(tuple(kv_cnt.shape) == (B, H, nqb) and tuple(kv_idx.shape) == (B, H, nqb, nkb),
              f"per-head lists are kv_cnt [{B}, {H}, {nqb}] and kv_idx [{B}, {H}, {nqb}, {nkb}]")


def _on_gpu(*tensors):
    """Last check before a call into the library: every tensor on one GPU."""
    ts = [t for t in tensors if t is not None]
    _need(all(t.is_cuda and t.device == ts[0].device for t in ts), "tensors must be on one GPU")


def geom_counts(sides, tile: int, q_scale: int):
    """(nqb, nkb, nq, nk) of a query scale (host only)."""
    g = make_geom(sides, tile)
    nqb, nkb = ctypes.c_int32(), ctypes.c_int32()
    nq, nk = ctypes.c_int64(), ctypes.c_int64()
    _check(_LIB.varsparse_geom_counts(ctypes.byref(g), q_scale, ctypes.byref(nqb), ctypes.byref(nkb),
                                      ctypes.byref(nq), ctypes.byref(nk)), "varsparse_geom_counts")
    return nqb.value, nkb.value, nq.value, nk.value


def window_radius(n_scales: int, q_scale: int, windows=(3, 5, 7)):
    """Per-key-scale radii of a query scale under the window schedule of the
    last len(windows) scales (host only)."""
    w = (ctypes.c_int32 * len(windows))(*[int(x) for x in windows])
    out = (ctypes.c_int32 * (q_scale + 1))()
    _check(_LIB.varsparse_window_radius(n_scales, q_scale, w, len(windows), out), "varsparse_window_radius")
    return list(out)


def build_mask(sides, tile: int, q_scale: int, n_sink: int, radius=None, budget: int = -1,
               want_mask: bool = False, device="cuda", out=None, stream=None):
    """CSLA kept-tile lists: (kv_cnt int32 [nqb], kv_idx int32 [nqb, nkb], mask uint8 [nqb, nkb] or None).
    ``out`` may pass preallocated (kv_cnt, kv_idx, mask)."""
    nqb, nkb, _, _ = geom_counts(sides, tile, q_scale)
    _need(radius is None or len(radius) >= q_scale + 1, "radius needs one entry per attended scale")
    if out is None:
        kv_cnt = torch.empty(nqb, dtype=torch.int32, device=device)
        kv_idx = torch.empty(nqb, nkb, dtype=torch.int32, device=device)
        mask = torch.empty(nqb, nkb, dtype=torch.uint8, device=device) if want_mask else None
    else:
        kv_cnt, kv_idx, mask = out
        _need(tuple(kv_cnt.shape) == (nqb,) and tuple(kv_idx.shape) == (nqb, nkb), "out lists have the wrong shape")
        _need(kv_cnt.dtype == torch.int32 and kv_idx.dtype == torch.int32 and kv_idx.is_contiguous(),
              "out lists are contiguous int32")
        _need(mask is None or (tuple(mask.shape) == (nqb, nkb) and mask.dtype == torch.uint8 and mask.is_contiguous()),
              "out mask is a contiguous uint8 [nqb, nkb] tensor")
    _on_gpu(kv_cnt, kv_idx, mask)
    g = make_geom(sides, tile)
    rad = None
    if radius is not None:
        rad = (ctypes.c_int32 * (q_scale + 1))(*[int(r) for r in radius[: q_scale + 1]])
    _check(_LIB.varsparse_build_mask(ctypes.byref(g), q_scale, n_sink, rad, budget, _ptr(mask),
                                     _ptr(kv_cnt), _ptr(kv_idx), _stream(stream)), "varsparse_build_mask")
    return kv_cnt, kv_idx, mask


def map_indices(sides, tile: int, d_scale: int, t_scale: int, n_sink: int, top_p: float,
                q_d=None, k=None, softmax_scale=None, scores=None, want_selection=False, out=None, stream=None,
                top_k=None):
    """CS4A: scores (computed when q_d is given, else taken from ``scores``),
    selection and per-(b,h) target lists.  Returns (scores, sel_cnt, sel_idx, kv_cnt, kv_idx).
    With ``top_k`` (a fraction in (0, 1]) the Top-K rule replaces top-p."""
    if q_d is not None:
        B, H, _, d = q_d.shape
        device = q_d.device
    else:
        B, H = scores.shape[:2]
        d = 0
        device = scores.device
    nqbD, nkbD, _, _ = geom_counts(sides, tile, d_scale)
    nqbT, nkbT, _, _ = geom_counts(sides, tile, t_scale)
    if scores is None:
        scores = torch.empty(B, H, nqbD, nkbD, dtype=torch.float32, device=device)
    if out is None:
        kv_cnt = torch.empty(B, H, nqbT, dtype=torch.int32, device=device)
        kv_idx = torch.empty(B, H, nqbT, nkbT, dtype=torch.int32, device=device)
    else:
        kv_cnt, kv_idx = out
    _need(tuple(scores.shape) == (B, H, nqbD, nkbD) and scores.dtype == torch.float32 and scores.is_contiguous(),
          f"scores is a contiguous float32 [{B}, {H}, {nqbD}, {nkbD}] tensor")
    _check_lists(kv_cnt, kv_idx, B, H, nqbT, nkbT)
    _need(kv_cnt.dim() == 3, "target lists are per (b, h)")
    if q_d is not None:
        _need(k is not None and k.dim() == 4 and tuple(k.shape[:2]) == (B, H) and k.shape[3] == d,
              "k must be [B, H, tokens, head_dim] like q_d")
        _need(q_d.shape[2] == geom_counts(sides, tile, d_scale)[2], "q_d must hold the decision scale's tokens")
        _need(k.shape[2] >= geom_counts(sides, tile, d_scale)[3], "k holds fewer tokens than the decision scale attends")
        _need(q_d.dtype == k.dtype, "q_d and k share one dtype")
    _on_gpu(q_d, k, scores, kv_cnt, kv_idx)
    sel_cnt = sel_idx = None
    if want_selection:
        sel_cnt = torch.empty(B, H, nqbD, dtype=torch.int32, device=device)
        sel_idx = torch.empty(B, H, nqbD, nkbD, dtype=torch.int32, device=device)
    g = make_geom(sides, tile)
    if q_d is not None:
        scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
        qs = (ctypes.c_int64 * 3)(*q_d.stride()[:3])
        ks = (ctypes.c_int64 * 3)(*k.stride()[:3])
        if q_d.stride(-1) != 1 or k.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
        dt = _dtype_code(q_d)
    else:
        scale, qs, ks, dt = 1.0, None, None, BF16
    fn, name, param = _LIB.varsparse_map_indices, "varsparse_map_indices", top_p
    if top_k is not None:
        fn, name, param = _LIB.varsparse_map_indices_topk, "varsparse_map_indices_topk", top_k
    _check(fn(ctypes.byref(g), d_scale, t_scale, n_sink, float(param), dt, B, H, d,
              _ptr(q_d), qs, _ptr(k), ks, float(scale), _ptr(scores),
              _ptr(sel_cnt), _ptr(sel_idx), _ptr(kv_cnt), _ptr(kv_idx), _stream(stream)), name)
    return scores, sel_cnt, sel_idx, kv_cnt, kv_idx


SELECT = {"top_p": 0, "top_k": 1}


def map_indices_multi(sides, tile: int, d_scale: int, t_scales, n_sink: int, param: float, rule: str = "top_p",
                      q_d=None, k=None, softmax_scale=None, scores=None, out=None, stream=None):
    """CS4A onto several target scales in one launch: scores (computed when q_d
    is given, else taken from ``scores``), then per target the lists
    map_indices would write.  Returns (scores, [(kv_cnt, kv_idx) per target])."""
    t_scales = [int(t) for t in t_scales]
    _need(1 <= len(t_scales) <= 8, "one to eight target scales")
    if q_d is not None:
        B, H, _, d = q_d.shape
        device = q_d.device
    else:
        B, H = scores.shape[:2]
        d = 0
        device = scores.device
    nqbD, nkbD, nqD, nkD = geom_counts(sides, tile, d_scale)
    if scores is None:
        scores = torch.empty(B, H, nqbD, nkbD, dtype=torch.float32, device=device)
    _need(tuple(scores.shape) == (B, H, nqbD, nkbD) and scores.dtype == torch.float32 and scores.is_contiguous(),
          f"scores is a contiguous float32 [{B}, {H}, {nqbD}, {nkbD}] tensor")
    if out is None:
        out = []
        for t in t_scales:
            nqbT, nkbT, _, _ = geom_counts(sides, tile, t)
            out.append((torch.empty(B, H, nqbT, dtype=torch.int32, device=device),
                        torch.empty(B, H, nqbT, nkbT, dtype=torch.int32, device=device)))
    _need(len(out) == len(t_scales), "one output pair per target scale")
    for t, (c, i) in zip(t_scales, out):
        nqbT, nkbT, _, _ = geom_counts(sides, tile, t)
        _check_lists(c, i, B, H, nqbT, nkbT)
        _need(c.dim() == 3, "target lists are per (b, h)")
    g = make_geom(sides, tile)
    if q_d is not None:
        _need(k is not None and k.dim() == 4 and tuple(k.shape[:2]) == (B, H) and k.shape[3] == d,
              "k must be [B, H, tokens, head_dim] like q_d")
        _need(q_d.shape[2] == nqD, "q_d must hold the decision scale's tokens")
        _need(k.shape[2] >= nkD, "k holds fewer tokens than the decision scale attends")
        _need(q_d.dtype == k.dtype, "q_d and k share one dtype")
        _need(q_d.stride(-1) == 1 and k.stride(-1) == 1, "the head dimension must be contiguous")
        scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
        qs = (ctypes.c_int64 * 3)(*q_d.stride()[:3])
        ks = (ctypes.c_int64 * 3)(*k.stride()[:3])
        dt = _dtype_code(q_d)
    else:
        scale, qs, ks, dt = 1.0, None, None, BF16
    _on_gpu(q_d, k, scores, *[x for pair in out for x in pair])
    n = len(t_scales)
    ts = (ctypes.c_int32 * n)(*t_scales)
    cnts = (ctypes.c_void_p * n)(*[c.data_ptr() for c, _ in out])
    idxs = (ctypes.c_void_p * n)(*[i.data_ptr() for _, i in out])
    _check(_LIB.varsparse_map_indices_multi(ctypes.byref(g), d_scale, n, ts, n_sink, SELECT[rule], float(param), dt,
                                            B, H, d, _ptr(q_d), qs, _ptr(k), ks, float(scale), _ptr(scores), cnts,
                                            idxs, _stream(stream)), "varsparse_map_indices_multi")
    return scores, list(out)


def attn_fwd(q, k, v, sides, tile: int, q_scale: int, kv_cnt, kv_idx, softmax_scale=None,
             out=None, lse=None, want_lse=True, stream=None):
    """Block-sparse attention; q [B,H,side^2,d], k/v [B,H,Nk,d].  Lists shared
    (kv_cnt [nqb]) or per (b,h) (kv_cnt [B,H,nqb]).  Returns (o, lse)."""
    B, H, nq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    nqb, nkb, nq_s, nk_s = geom_counts(sides, tile, q_scale)
    _check_qkvo(q, k, v, out, lse, nq_s, nk_s, bf16_only=False)
    _check_lists(kv_cnt, kv_idx, B, H, nqb, nkb)
    _on_gpu(q, k, v, out, lse, kv_cnt, kv_idx)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    per_head = 1 if kv_cnt.dim() == 3 else 0
    g = make_geom(sides, tile)
    _check(_LIB.varsparse_attn_fwd(ctypes.byref(g), q_scale, _dtype_code(q), B, H, d, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(out), _ptr(lse), _strides(q, k, v, out), float(scale), _ptr(kv_cnt),
                                   _ptr(kv_idx), per_head, _stream(stream)), "varsparse_attn_fwd")
    return out, lse


def attn_fwd_pair(q, k, v, sides, tile: int, q_scale: int, kv_cnt, kv_idx, softmax_scale=None,
                  out=None, lse=None, want_lse=True, stream=None):
    """Block-sparse attention with 128-query workgroups over pairs of query
    tiles (bf16); same arguments and results as attn_fwd.  Returns (o, lse)."""
    B, H, nq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    nqb, nkb, nq_s, nk_s = geom_counts(sides, tile, q_scale)
    _check_qkvo(q, k, v, out, lse, nq_s, nk_s, bf16_only=True)
    _check_lists(kv_cnt, kv_idx, B, H, nqb, nkb)
    _on_gpu(q, k, v, out, lse, kv_cnt, kv_idx)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    per_head = 1 if kv_cnt.dim() == 3 else 0
    g = make_geom(sides, tile)
    _check(_LIB.varsparse_attn_fwd_pair(ctypes.byref(g), q_scale, B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(lse), _strides(q, k, v, out), float(scale), _ptr(kv_cnt), _ptr(kv_idx),
                                        per_head, _stream(stream)), "varsparse_attn_fwd_pair")
    return out, lse


def attn_fwd_ocache(q, k, v, sides, tile: int, q_scale: int, kv_cnt, kv_idx, d_scale: int, o_full_d, o_sparse_d,
                    softmax_scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Block-sparse attention of a later scale with the O_cache correction
    added before the output's rounding: attn_fwd followed by ocache_correct
    in one pass (bf16).  o_full_d / o_sparse_d: the decision scale's full and
    block-sparse outputs [B,H,side_d^2,d].  Returns (o, lse)."""
    B, H, nq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    nqb, nkb, nq_s, nk_s = geom_counts(sides, tile, q_scale)
    _check_qkvo(q, k, v, out, lse, nq_s, nk_s, bf16_only=True)
    _check_lists(kv_cnt, kv_idx, B, H, nqb, nkb)
    _need(0 <= d_scale <= q_scale, "the decision scale is at or below the query scale")
    nd = geom_counts(sides, tile, d_scale)[2]
    for name, t in (("o_full_d", o_full_d), ("o_sparse_d", o_sparse_d)):
        _need(tuple(t.shape) == (B, H, nd, d) and t.dtype == torch.bfloat16,
              f"{name} is a bfloat16 [{B}, {H}, {nd}, {d}] tensor")
        _need(t.stride(-1) == 1, "the head dimension must be contiguous")
    _on_gpu(q, k, v, out, lse, kv_cnt, kv_idx, o_full_d, o_sparse_d)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    per_head = 1 if kv_cnt.dim() == 3 else 0
    g = make_geom(sides, tile)
    ds = (ctypes.c_int64 * 6)(*o_full_d.stride()[:3], *o_sparse_d.stride()[:3])
    _check(_LIB.varsparse_attn_fwd_ocache(ctypes.byref(g), q_scale, d_scale, B, H, d, _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(out), _ptr(lse), _strides(q, k, v, out), float(scale), _ptr(kv_cnt),
                                          _ptr(kv_idx), per_head, _ptr(o_full_d), _ptr(o_sparse_d), ds,
                                          _stream(stream)), "varsparse_attn_fwd_ocache")
    return out, lse


def attn_fwd_multi(qs, k, v, sides, tile: int, q_scales, lists, softmax_scale=None, outs=None, lses=None,
                   want_lse=True, d_scale=None, o_full_d=None, o_sparse_d=None, stream=None):
    """Block-sparse attention of several query scales over one cache in one
    launch (bf16): target i is what attn_fwd (or, with the decision outputs
    o_full_d / o_sparse_d of d_scale, attn_fwd_ocache) returns for q_scales[i],
    qs[i] and lists[i] = (kv_cnt, kv_idx).  Returns [(o, lse) per target]."""
    q_scales = [int(t) for t in q_scales]
    n = len(q_scales)
    _need(1 <= n <= MAX_ATTN_TARGETS, f"one to {MAX_ATTN_TARGETS} target scales")
    _need(len(qs) == n and len(lists) == n, "one query tensor and one list pair per target")
    B, H, _, d = qs[0].shape
    if outs is None:
        outs = [torch.empty_like(q) for q in qs]
    if lses is None:
        lses = [torch.empty(B, H, q.shape[2], dtype=torch.float32, device=q.device) if want_lse else None
                for q in qs]
    _need(len(outs) == n and len(lses) == n, "one output and one lse (or None) per target")
    per_head = 1 if lists[0][0].dim() == 3 else 0
    oc = o_full_d is not None or o_sparse_d is not None
    strides = []
    for t, q, out, lse, (c, i) in zip(q_scales, qs, outs, lses, lists):
        nqb, nkb, nq_s, nk_s = geom_counts(sides, tile, t)
        _need(q.shape[0] == B and q.shape[1] == H and q.shape[3] == d, "every target has q's B, H and head_dim")
        _check_qkvo(q, k, v, out, lse, nq_s, nk_s, bf16_only=True)
        _check_lists(c, i, B, H, nqb, nkb)
        _need((1 if c.dim() == 3 else 0) == per_head, "lists all shared or all per (b, h)")
        strides.extend(_strides(q, k, v, out))
        if oc:
            _need(d_scale is not None and 0 <= d_scale <= t, "the decision scale is at or below every target")
    ds = None
    if oc:
        _need(o_full_d is not None and o_sparse_d is not None, "both decision-scale outputs, or neither")
        nd = geom_counts(sides, tile, d_scale)[2]
        for name, t in (("o_full_d", o_full_d), ("o_sparse_d", o_sparse_d)):
            _need(tuple(t.shape) == (B, H, nd, d) and t.dtype == torch.bfloat16,
                  f"{name} is a bfloat16 [{B}, {H}, {nd}, {d}] tensor")
            _need(t.stride(-1) == 1, "the head dimension must be contiguous")
        ds = (ctypes.c_int64 * 6)(*o_full_d.stride()[:3], *o_sparse_d.stride()[:3])
    _on_gpu(*qs, k, v, *outs, *lses, *[x for pair in lists for x in pair], o_full_d, o_sparse_d)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    g = make_geom(sides, tile)
    ptrs = lambda ts: (ctypes.c_void_p * n)(*[None if t is None else t.data_ptr() for t in ts])
    _check(_LIB.varsparse_attn_fwd_multi(ctypes.byref(g), n, (ctypes.c_int32 * n)(*q_scales), B, H, d, ptrs(qs),
                                         _ptr(k), _ptr(v), ptrs(outs), ptrs(lses), (ctypes.c_int64 * len(strides))(*strides),
                                         float(scale), ptrs([c for c, _ in lists]), ptrs([i for _, i in lists]),
                                         per_head, -1 if d_scale is None else int(d_scale), _ptr(o_full_d),
                                         _ptr(o_sparse_d), ds, _stream(stream)), "varsparse_attn_fwd_multi")
    return list(zip(outs, lses))


def attn_fwd_token(q, k, v, sides, tile: int, q_scale: int, n_sink: int, radius, kv_cnt=None, kv_idx=None,
                   softmax_scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Token-exact CSLA attention (the token-level sink + window mask); with
    lists only their tiles are walked, without every key tile (the token-masked
    dense baseline).  Returns (o, lse)."""
    B, H, nq, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    nqb, nkb, nq_s, nk_s = geom_counts(sides, tile, q_scale)
    _check_qkvo(q, k, v, out, lse, nq_s, nk_s, bf16_only=True)
    _need((kv_cnt is None) == (kv_idx is None), "pass both lists or neither")
    if kv_cnt is not None:
        _check_lists(kv_cnt, kv_idx, B, H, nqb, nkb)
    _need(len(radius) >= q_scale + 1, "radius needs one entry per attended scale")
    _on_gpu(q, k, v, out, lse, kv_cnt, kv_idx)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    per_head = 1 if (kv_cnt is not None and kv_cnt.dim() == 3) else 0
    rad = (ctypes.c_int32 * (q_scale + 1))(*[int(r) for r in radius[: q_scale + 1]])
    g = make_geom(sides, tile)
    _check(_LIB.varsparse_attn_fwd_token(ctypes.byref(g), q_scale, n_sink, rad, B, H, d, _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(out), _ptr(lse), _strides(q, k, v, out), float(scale), _ptr(kv_cnt),
                                         _ptr(kv_idx), per_head, _stream(stream)), "varsparse_attn_fwd_token")
    return out, lse


def dense_attn_fwd(q, k, v, softmax_scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Dense attention with the same tile engine; q [B,H,nq,d], k/v [B,H,nk,d]."""
    B, H, nq, d = q.shape
    nk = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, H, nq, dtype=torch.float32, device=q.device)
    _check_qkvo(q, k, v, out, lse, nq, nk, bf16_only=False)
    _need(v.shape[2] >= nk, "v holds fewer tokens than k")
    _on_gpu(q, k, v, out, lse)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    _check(_LIB.varsparse_dense_attn_fwd(_dtype_code(q), B, H, d, nq, nk, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                         _ptr(lse), _strides(q, k, v, out), float(scale), _stream(stream)),
           "varsparse_dense_attn_fwd")
    return out, lse


def dense_attn_fwd_multi(qs, k, v, nks, softmax_scale=None, outs=None, lses=None, want_lse=True, stream=None):
    """Dense attention of several query sets over prefixes of one cache in one
    launch (bf16): target i is the attention dense_attn_fwd computes for
    qs[i] over k[:, :, :nks[i]], v[:, :, :nks[i]], each 64-query block walked
    in one pass.  Returns [(o, lse) per target]."""
    n = len(qs)
    _need(1 <= n <= MAX_DENSE_TARGETS and len(nks) == n, f"one to {MAX_DENSE_TARGETS} query sets, one length each")
    B, H, _, d = qs[0].shape
    if outs is None:
        outs = [torch.empty_like(q) for q in qs]
    if lses is None:
        lses = [torch.empty(B, H, q.shape[2], dtype=torch.float32, device=q.device) if want_lse else None
                for q in qs]
    _need(len(outs) == n and len(lses) == n, "one output and one lse (or None) per target")
    strides = []
    for q, out, lse, nk in zip(qs, outs, lses, nks):
        _need(q.dim() == 4 and q.shape[0] == B and q.shape[1] == H and q.shape[3] == d,
              "every query set is [B, H, nq, head_dim] with the first's B, H and head_dim")
        _need(1 <= int(nk), "every target attends at least one key")
        _check_qkvo(q, k, v, out, lse, q.shape[2], int(nk), bf16_only=True)
        strides.extend(_strides(q, k, v, out))
    _on_gpu(*qs, k, v, *outs, *lses)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    ptrs = lambda ts: (ctypes.c_void_p * n)(*[None if t is None else t.data_ptr() for t in ts])
    i64 = lambda vals: (ctypes.c_int64 * n)(*[int(x) for x in vals])
    _check(_LIB.varsparse_dense_attn_fwd_multi(n, B, H, d, i64([q.shape[2] for q in qs]), i64(nks), ptrs(qs), _ptr(k),
                                               _ptr(v), ptrs(outs), ptrs(lses),
                                               (ctypes.c_int64 * len(strides))(*strides), float(scale),
                                               _stream(stream)), "varsparse_dense_attn_fwd_multi")
    return list(zip(outs, lses))


def ocache_correct(o_full_d, o_sparse_d, o_t, side_d: int, side_t: int, stream=None):
    """O_cache: o_t += nearest-upsampled (o_full_d - o_sparse_d), in place.
    o_full_d / o_sparse_d [B,H,side_d^2,d], o_t [B,H,side_t^2,d], bf16."""
    B, H, nt, d = o_t.shape
    if o_full_d.shape != o_sparse_d.shape or o_full_d.shape[:2] != (B, H) or o_full_d.shape[3] != d:
        raise ValueError("shape mismatch between the decision outputs and the target output")
    if o_full_d.shape[2] != side_d * side_d or nt != side_t * side_t:
        raise ValueError("token counts do not match the sides")
    if any(t.stride(-1) != 1 for t in (o_full_d, o_sparse_d, o_t)):
        raise ValueError("the head dimension must be contiguous")
    _need(all(t.dtype == torch.bfloat16 for t in (o_full_d, o_sparse_d, o_t)), "O_cache tensors are bfloat16")
    _on_gpu(o_full_d, o_sparse_d, o_t)
    st = (ctypes.c_int64 * 9)(*o_full_d.stride()[:3], *o_sparse_d.stride()[:3], *o_t.stride()[:3])
    _check(_LIB.varsparse_ocache_correct(B, H, d, side_d, side_t, _ptr(o_full_d), _ptr(o_sparse_d), _ptr(o_t), st,
                                         _stream(stream)), "varsparse_ocache_correct")
    return o_t


JOIN = {"union": 0, "intersection": 1}


def join_lists(a_cnt, a_idx, b_cnt, b_idx, join: str = "union", out=None, stream=None):
    """Per-row union or intersection of two ascending kept-tile lists.

    Lists are int32 cnt [..., rows] / idx [..., rows, nkb] on the device; a
    list set without leading dimensions is shared by every set of the other.
    Returns (cnt, idx) with the leading shape of the per-set input."""
    for x in (a_cnt, a_idx, b_cnt, b_idx):
        if x.dtype != torch.int32 or not x.is_contiguous():
            raise ValueError("lists are contiguous int32 tensors")
    rows, nkb = a_idx.shape[-2], a_idx.shape[-1]
    if b_idx.shape[-2:] != (rows, nkb) or a_cnt.shape[-1] != rows or b_cnt.shape[-1] != rows:
        raise ValueError("list shapes differ")
    if a_cnt.shape[:-1] != a_idx.shape[:-2] or b_cnt.shape[:-1] != b_idx.shape[:-2]:
        raise ValueError("cnt and idx leading shapes differ")
    lead_a, lead_b = tuple(a_cnt.shape[:-1]), tuple(b_cnt.shape[:-1])
    if lead_a and lead_b and lead_a != lead_b:
        raise ValueError("per-set lists of both sides must have the same leading shape")
    lead = lead_a or lead_b
    sets = math.prod(lead) if lead else 1
    if out is None:
        out = (torch.empty(*lead, rows, dtype=torch.int32, device=a_cnt.device),
               torch.empty(*lead, rows, nkb, dtype=torch.int32, device=a_cnt.device))
    oc, oi = out
    if tuple(oc.shape) != (*lead, rows) or tuple(oi.shape) != (*lead, rows, nkb):
        raise ValueError("output shape")
    _check(_LIB.varsparse_join_lists(sets, rows, nkb, JOIN[join], _ptr(a_cnt), _ptr(a_idx), int(bool(lead_a)),
                                     _ptr(b_cnt), _ptr(b_idx), int(bool(lead_b)), _ptr(oc), _ptr(oi),
                                     _stream(stream)), "varsparse_join_lists")
    return oc, oi

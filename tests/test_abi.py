"""The C ABI without a GPU: the library loads, exports every function the
header declares, computes counts on the host, and rejects malformed or
unsupported arguments before touching HIP.  Every call here either fails
validation or has an empty batch, so none of them launches anything."""
import ctypes
import os
import re

import pytest

vs = pytest.importorskip("block_sparse_cross_csla_amd")
from block_sparse_cross_csla_amd import _lib  # noqa: E402
from varsparse_inputs import SCHEDULE_13, SCHEDULE_16, TINY_SIDES  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "varsparse.h")


def test_exports_every_declared_function():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(varsparse_\w+)\s*\(", text, re.M))
    assert declared == set(_lib.EXPORTS)
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_geom_counts():
    assert vs.geom_counts(SCHEDULE_13, 8, 12) == (64, 172, 4096, 10521)
    assert vs.geom_counts(SCHEDULE_13, 8, 9) == (16, 47, 1024, 2521)
    assert vs.geom_counts(TINY_SIDES, 4, 4) == (16, 23, 256, 341)
    assert vs.geom_counts(SCHEDULE_16, 8, 15) == (256, 672, 16384, 42521)


def test_strerror():
    lib = _lib.lib()
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-2, b"unsupported configuration"),
                       (-3, b"HIP launch error")]:
        assert lib.varsparse_strerror(code) == text
    assert lib.varsparse_last_hip_error() == 0


def _g(sides=SCHEDULE_13, tile=8):
    return ctypes.byref(_lib.make_geom(sides, tile))


FAKE = ctypes.c_void_p(1 << 20)       # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)
I32 = ctypes.c_int32


def _strides(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


GOOD12 = [0, 0, 128] * 4


@pytest.mark.parametrize("sides,tile", [((), 8), ((4, 4), 8), ((4, 2), 8), ((0, 4), 8), ((2, 4), 0)])
def test_bad_geometry(sides, tile):
    lib = _lib.lib()
    assert lib.varsparse_geom_counts(_g(sides, tile), 0, None, None, None, None) == _lib.EINVAL


def test_build_mask_validation():
    lib = _lib.lib()
    rad = (I32 * 13)(*([2] * 13))
    call = lambda **kw: lib.varsparse_build_mask(  # noqa: E731
        kw.get("g", _g()), kw.get("q", 12), kw.get("n_sink", 5), kw.get("rad", rad), kw.get("budget", -1),
        None, kw.get("cnt", FAKE), kw.get("idx", FAKE), None)
    assert call(q=13) == _lib.EINVAL                      # query scale out of range
    assert call(q=-1) == _lib.EINVAL
    assert call(n_sink=13) == _lib.EINVAL                 # more sinks than earlier scales
    assert call(n_sink=-1) == _lib.EINVAL
    assert call(budget=0) == _lib.EINVAL
    assert call(budget=-2) == _lib.EINVAL
    assert call(rad=None) == _lib.EINVAL                  # radius mode needs radii
    assert call(cnt=None) == _lib.EINVAL
    assert call(idx=None) == _lib.EINVAL
    assert call(g=_g(SCHEDULE_13, 7)) == _lib.EINVAL      # side 64 not a multiple of the tile


def test_attn_validation():
    lib = _lib.lib()

    def call(**kw):
        return lib.varsparse_attn_fwd(
            kw.get("g", _g()), kw.get("q", 12), kw.get("dt", _lib.BF16), kw.get("B", 2), kw.get("H", 16),
            kw.get("d", 128), kw.get("qp", FAKE), FAKE, FAKE, FAKE, None, _strides(kw.get("st", GOOD12)),
            kw.get("scale", 0.088), FAKE, FAKE, kw.get("per_head", 0), None)
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(d=256) == _lib.EUNSUPPORTED
    assert call(g=_g(SCHEDULE_13, 4)) == _lib.EUNSUPPORTED    # bf16 MFMA path uses 8x8 tiles
    assert call(g=_g(TINY_SIDES, 16), q=4, dt=_lib.FP32, d=64) == _lib.EUNSUPPORTED
    assert call(dt=7) == _lib.EINVAL
    # K or V rows 2^20 elements apart over 10521 cached tokens: byte offsets past
    # 2^31, which the bf16 kernels cannot address (32-bit per-head offsets)
    far = 1 << 20
    assert call(st=[0, 0, 128, 0, 0, far, 0, 0, 128, 0, 0, 128]) == _lib.EUNSUPPORTED
    assert call(st=[0, 0, 128, 0, 0, 128, 0, 0, far, 0, 0, 128]) == _lib.EUNSUPPORTED
    assert call(B=-1) == _lib.EINVAL
    assert call(H=-1) == _lib.EINVAL
    assert call(scale=0.0) == _lib.EINVAL
    assert call(scale=float("nan")) == _lib.EINVAL
    assert call(qp=None) == _lib.EINVAL
    assert call(qp=MISALIGNED) == _lib.EINVAL
    assert call(st=[0, 0, 132] + GOOD12[3:]) == _lib.EINVAL   # bf16 rows not 16-byte aligned
    assert call(per_head=2) == _lib.EINVAL
    assert call(q=13) == _lib.EINVAL


def test_dense_validation():
    lib = _lib.lib()

    def call(**kw):
        return lib.varsparse_dense_attn_fwd(kw.get("dt", _lib.BF16), 1, 1, kw.get("d", 128), kw.get("nq", 10),
                                            kw.get("nk", 10), FAKE, FAKE, FAKE, FAKE, None,
                                            _strides(GOOD12), kw.get("scale", 0.1), None)
    assert call(nq=-1) == _lib.EINVAL
    assert call(nk=0) == _lib.EINVAL
    assert call(d=32) == _lib.EUNSUPPORTED
    assert call(scale=-1.0) == _lib.EINVAL
    assert call(nk=1 << 31) == _lib.EUNSUPPORTED


def test_map_indices_validation():
    lib = _lib.lib()

    def call(**kw):
        return lib.varsparse_map_indices(
            _g(), kw.get("D", 9), kw.get("T", 12), kw.get("n_sink", 5), kw.get("p", 0.9), _lib.BF16, 2, 16,
            kw.get("d", 128), kw.get("qd", None), None, None, None, 0.1, kw.get("scores", FAKE),
            kw.get("sel_cnt", None), None, FAKE, FAKE, None)
    assert call(D=13) == _lib.EINVAL
    assert call(D=10, T=9) == _lib.EINVAL
    assert call(n_sink=10) == _lib.EINVAL
    assert call(p=0.0) == _lib.EINVAL
    assert call(p=1.5) == _lib.EINVAL
    assert call(scores=None) == _lib.EINVAL
    assert call(sel_cnt=FAKE) == _lib.EINVAL             # selection outputs come in pairs
    assert call(qd=FAKE) == _lib.EINVAL                  # scoring needs k and strides
    assert call(qd=FAKE, d=96) == _lib.EUNSUPPORTED


def test_ocache_validation():
    lib = _lib.lib()
    st = (ctypes.c_int64 * 9)(*([128 * 1024, 1024 * 128, 128] * 3))
    p = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced: validation fails first
    call = lambda B=1, H=1, d=128, sd=32, stt=64, f=p, sp=p, o=p, strides=st: lib.varsparse_ocache_correct(
        B, H, d, sd, stt, f, sp, o, strides, None)
    assert call(B=-1) == _lib.EINVAL
    assert call(H=-1) == _lib.EINVAL
    assert call(d=12) == _lib.EINVAL                 # not a multiple of 8
    assert call(sd=0) == _lib.EINVAL
    assert call(sd=64, stt=32) == _lib.EINVAL        # target smaller than the decision scale
    assert call(f=None) == _lib.EINVAL
    assert call(o=ctypes.c_void_p((1 << 20) + 8)) == _lib.EINVAL   # misaligned
    bad = (ctypes.c_int64 * 9)(*([128 * 1024, 1024 * 128, 130] * 3))
    assert call(strides=bad) == _lib.EINVAL          # token stride not a multiple of 8


def test_join_validation():
    lib = _lib.lib()
    p, q, o1, o2 = (ctypes.c_void_p((1 << 20) + 4096 * i) for i in range(4))

    def call(sets=2, rows=64, nkb=172, join=0, ac=p, ai=q, bc=p, bi=q, oc=o1, oi=o2):
        return lib.varsparse_join_lists(sets, rows, nkb, join, ac, ai, 1, bc, bi, 0, oc, oi, None)

    assert call(sets=-1) == _lib.EINVAL
    assert call(rows=0) == _lib.EINVAL
    assert call(nkb=0) == _lib.EINVAL
    assert call(nkb=65537) == _lib.EINVAL
    assert call(join=2) == _lib.EINVAL
    assert call(sets=1 << 16, rows=1 << 15) == _lib.EINVAL      # 2^31 rows
    assert call(ai=None) == _lib.EINVAL
    assert call(oc=None) == _lib.EINVAL
    assert call(oi=q) == _lib.EINVAL                             # output aliases an input


def test_window_radius_matches_oracle():
    from oracle import schedule as S
    for n, windows in ((13, (3, 5, 7)), (16, (3, 5, 7)), (16, (9,)), (5, (1, 3))):
        for q in range(n - len(windows), n):
            assert vs.window_radius(n, q, windows) == S.window_radius(n, q, windows)
    lib = _lib.lib()
    w = (ctypes.c_int32 * 3)(3, 5, 7)
    out = (ctypes.c_int32 * 16)()
    for args in ((13, 9, w, 3), (13, 12, w, 0), (13, 12, w, 14), (0, 0, w, 1), (33, 32, w, 3), (13, 12, None, 3)):
        assert lib.varsparse_window_radius(*args, out) == _lib.EINVAL
    even = (ctypes.c_int32 * 3)(3, 4, 7)
    assert lib.varsparse_window_radius(13, 11, even, 3, out) == _lib.EINVAL
    assert lib.varsparse_window_radius(13, 11, w, 3, None) == _lib.EINVAL


def test_attn_token_validation():
    lib = _lib.lib()
    rad = (ctypes.c_int32 * 32)(*([2] * 32))

    def call(**kw):
        return lib.varsparse_attn_fwd_token(
            kw.get("g", _g()), kw.get("q", 12), kw.get("sink", 5), kw.get("rad", rad), kw.get("B", 2),
            kw.get("H", 16), kw.get("d", 128), FAKE, FAKE, FAKE, FAKE, None, _strides(GOOD12),
            kw.get("scale", 0.088), kw.get("cnt", FAKE), kw.get("idx", FAKE), 0, None)
    assert call(sink=-1) == _lib.EINVAL
    assert call(sink=13) == _lib.EINVAL                       # more sinks than attended scales
    assert call(rad=None) == _lib.EINVAL
    assert call(cnt=None) == _lib.EINVAL                      # lists: both or neither
    assert call(idx=None) == _lib.EINVAL
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(g=_g(SCHEDULE_13, 4)) == _lib.EUNSUPPORTED    # 8x8 tiles only
    big = (1, 2, 4, 8, 4104)                                  # query side above 4096
    assert call(g=_g(big), q=4, sink=2) == _lib.EUNSUPPORTED


def test_attn_pair_validation():
    lib = _lib.lib()

    def call(**kw):
        return lib.varsparse_attn_fwd_pair(
            kw.get("g", _g()), kw.get("q", 12), kw.get("B", 2), kw.get("H", 16), kw.get("d", 128),
            kw.get("qp", FAKE), FAKE, FAKE, FAKE, None, _strides(kw.get("st", GOOD12)), kw.get("scale", 0.088),
            kw.get("cnt", FAKE), FAKE, kw.get("per_head", 0), None)
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(g=_g(SCHEDULE_13, 4)) == _lib.EUNSUPPORTED    # 8x8 tiles only
    assert call(B=-1) == _lib.EINVAL
    assert call(scale=0.0) == _lib.EINVAL
    assert call(qp=None) == _lib.EINVAL
    assert call(cnt=None) == _lib.EINVAL
    assert call(qp=MISALIGNED) == _lib.EINVAL
    assert call(per_head=2) == _lib.EINVAL
    assert call(q=13) == _lib.EINVAL
    big = (8, 16, 32, 64, 128, 256, 512)                      # 5461 key tiles
    assert call(g=_g(big), q=6) == _lib.EUNSUPPORTED


def test_map_indices_multi_validation():
    lib = _lib.lib()
    p = ctypes.c_void_p(1 << 20)
    ptrs = (ctypes.c_void_p * 3)(p, p, p)
    nulls = (ctypes.c_void_p * 3)(p, None, p)

    def call(d=9, ts=(10, 11, 12), n=None, sink=5, rule=0, param=0.9, cnts=ptrs, idxs=ptrs, scores=p):
        n = len(ts) if n is None else n
        t = (ctypes.c_int32 * max(len(ts), 1))(*ts)
        return lib.varsparse_map_indices_multi(_g(), d, n, t, sink, rule, param, _lib.BF16, 2, 16, 128, None, None,
                                               None, None, 0.088, scores, cnts, idxs, None)
    assert call(n=0) == _lib.EINVAL
    assert call(n=9) == _lib.EINVAL                      # at most eight targets
    assert call(ts=(8, 11, 12)) == _lib.EINVAL           # a target below the decision scale
    assert call(ts=(10, 13, 12)) == _lib.EINVAL          # a target past the schedule
    assert call(rule=2) == _lib.EINVAL
    assert call(param=0.0) == _lib.EINVAL
    assert call(cnts=nulls) == _lib.EINVAL
    assert call(scores=None) == _lib.EINVAL
    assert call(sink=10) == _lib.EINVAL


def test_empty_batch_is_a_no_op():
    """B == 0 or H == 0 (dense: also nq == 0; join: sets == 0) returns OK with
    every data pointer NULL once the geometry and scalars pass, so nothing is
    read or enqueued; the same calls with a bad scalar still fail."""
    lib = _lib.lib()
    rad = (I32 * 32)(*([2] * 32))
    st12 = _strides(GOOD12)
    for B, H in ((0, 16), (2, 0), (0, 0)):
        assert lib.varsparse_attn_fwd(_g(), 12, _lib.BF16, B, H, 128, None, None, None, None, None, None, 0.088,
                                      None, None, 0, None) == _lib.OK
        assert lib.varsparse_attn_fwd(_g(), 12, _lib.BF16, B, H, 128, None, None, None, None, None, None, 0.0,
                                      None, None, 0, None) == _lib.EINVAL
        assert lib.varsparse_attn_fwd(_g(), 12, _lib.BF16, B, H, 96, None, None, None, None, None, None, 0.088,
                                      None, None, 0, None) == _lib.EUNSUPPORTED
        assert lib.varsparse_attn_fwd_pair(_g(), 12, B, H, 128, None, None, None, None, None, None, 0.088, None,
                                           None, 0, None) == _lib.OK
        assert lib.varsparse_attn_fwd_token(_g(), 12, 5, rad, B, H, 128, None, None, None, None, None, None,
                                            0.088, None, None, 0, None) == _lib.OK
        assert lib.varsparse_attn_fwd_token(_g(), 12, 13, rad, B, H, 128, None, None, None, None, None, st12,
                                            0.088, None, None, 0, None) == _lib.EINVAL
        assert lib.varsparse_dense_attn_fwd(_lib.BF16, B, H, 128, 10, 10, None, None, None, None, None, None,
                                            0.088, None) == _lib.OK
        assert lib.varsparse_ocache_correct(B, H, 128, 32, 64, None, None, None, None, None) == _lib.OK
        assert lib.varsparse_map_indices(_g(), 9, 12, 5, 0.9, _lib.BF16, B, H, 128, None, None, None, None, 0.088,
                                         None, None, None, None, None, None) == _lib.OK
        assert lib.varsparse_map_indices(_g(), 9, 12, 5, 0.0, _lib.BF16, B, H, 128, None, None, None, None, 0.088,
                                         None, None, None, None, None, None) == _lib.EINVAL
        assert lib.varsparse_map_indices_topk(_g(), 9, 12, 5, 0.2, _lib.BF16, B, H, 128, None, None, None, None,
                                              0.088, None, None, None, None, None, None) == _lib.OK
        ts = (I32 * 2)(10, 12)
        nulls = (ctypes.c_void_p * 2)(None, None)
        assert lib.varsparse_map_indices_multi(_g(), 9, 2, ts, 5, 0, 0.9, _lib.BF16, B, H, 128, None, None, None,
                                               None, 0.088, None, nulls, nulls, None) == _lib.OK
    assert lib.varsparse_dense_attn_fwd(_lib.BF16, 1, 1, 128, 0, 10, None, None, None, None, None, None,
                                        0.088, None) == _lib.OK
    assert lib.varsparse_join_lists(0, 64, 172, 0, None, None, 1, None, None, 0, None, None, None) == _lib.OK
    assert lib.varsparse_join_lists(0, 64, 172, 2, None, None, 1, None, None, 0, None, None, None) == _lib.EINVAL


def test_attn_ocache_validation():
    lib = _lib.lib()
    d6 = _strides([0, 0, 128] * 2)

    def call(**kw):
        return lib.varsparse_attn_fwd_ocache(
            kw.get("g", _g()), kw.get("q", 12), kw.get("D", 9), kw.get("B", 2), kw.get("H", 16), kw.get("d", 128),
            FAKE, FAKE, FAKE, FAKE, None, _strides(GOOD12), kw.get("scale", 0.088), FAKE, FAKE,
            kw.get("per_head", 1), kw.get("f", FAKE), kw.get("p", FAKE), _strides(kw.get("ds", [0, 0, 128] * 2)),
            None)
    assert call(D=13) == _lib.EINVAL                          # decision scale above the query scale
    assert call(D=-1) == _lib.EINVAL
    assert call(f=None) == _lib.EINVAL
    assert call(p=MISALIGNED) == _lib.EINVAL
    assert call(ds=[0, 0, 130, 0, 0, 128]) == _lib.EINVAL    # decision rows not 16-byte aligned
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(g=_g(SCHEDULE_13, 4)) == _lib.EUNSUPPORTED    # 8x8 tiles only
    assert call(B=-1) == _lib.EINVAL
    assert call(per_head=2) == _lib.EINVAL
    assert lib.varsparse_attn_fwd_ocache(_g(), 12, 9, 0, 16, 128, None, None, None, None, None, None, 0.088, None,
                                         None, 0, None, None, d6, None) == _lib.OK     # empty batch


def test_attn_multi_validation():
    lib = _lib.lib()
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)

    def call(**kw):
        n = kw.get("n", 3)
        ts = kw.get("ts", [12, 11, 10][:max(n, 0)] or [12])
        st = kw.get("st", GOOD12 * max(n, 1))
        return lib.varsparse_attn_fwd_multi(
            kw.get("g", _g()), n, (I32 * len(ts))(*ts), kw.get("B", 2), 16, kw.get("d", 128),
            arr(*([kw.get("qp", FAKE)] * len(ts))), FAKE, FAKE, arr(*([FAKE] * len(ts))), None, _strides(st),
            0.088, arr(*([FAKE] * len(ts))), arr(*([FAKE] * len(ts))), kw.get("per_head", 1), kw.get("D", 9),
            kw.get("f", None), kw.get("p", None), _strides([0, 0, 128] * 2), None)
    assert call(n=0) == _lib.EINVAL
    assert call(n=4, ts=[12, 11, 10, 9]) == _lib.EINVAL          # more targets than one launch carries
    assert call(ts=[12, 11, 13]) == _lib.EINVAL
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(g=_g(SCHEDULE_13, 4)) == _lib.EUNSUPPORTED        # 8x8 tiles only
    assert call(per_head=2) == _lib.EINVAL
    assert call(qp=MISALIGNED) == _lib.EINVAL
    assert call(qp=None) == _lib.EINVAL
    other_k = GOOD12 * 2 + [0, 0, 128, 0, 0, 256] + GOOD12[6:]
    assert call(st=other_k) == _lib.EINVAL                        # one cache: K strides equal for every target
    assert call(f=FAKE, p=None) == _lib.EINVAL                    # both decision outputs or neither
    assert call(f=FAKE, p=FAKE, D=11) == _lib.EINVAL              # decision scale above target 10
    assert call(B=0) == _lib.OK                                   # empty batch


def test_dense_multi_validation():
    lib = _lib.lib()
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    i64 = lambda *v: (ctypes.c_int64 * len(v))(*v)

    def call(**kw):
        nq = kw.get("nq", [64, 256])
        n = kw.get("n", len(nq))
        nk = kw.get("nk", [121, 341])
        return lib.varsparse_dense_attn_fwd_multi(
            n, kw.get("B", 2), 16, kw.get("d", 128), i64(*nq), i64(*nk), arr(*([kw.get("qp", FAKE)] * len(nq))),
            FAKE, FAKE, arr(*([FAKE] * len(nq))), None, _strides(kw.get("st", GOOD12 * len(nq))), 0.088, None)
    assert call(n=0) == _lib.EINVAL
    assert call(n=17, nq=[64] * 17, nk=[64] * 17) == _lib.EINVAL    # more query sets than one launch carries
    assert call(nk=[121, 0]) == _lib.EINVAL
    assert call(nq=[64, -1]) == _lib.EINVAL
    assert call(nk=[121, 1 << 30]) == _lib.EUNSUPPORTED
    assert call(d=96) == _lib.EUNSUPPORTED
    assert call(qp=MISALIGNED) == _lib.EINVAL
    assert call(qp=None) == _lib.EINVAL
    assert call(st=GOOD12 + [0, 0, 128, 0, 0, 256] + GOOD12[6:]) == _lib.EINVAL   # one cache: K strides equal
    assert call(B=0) == _lib.OK                                                  # empty batch
    assert call(nq=[0, 0], qp=None) == _lib.OK                                   # no queries at all

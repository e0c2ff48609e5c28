"""Block-sparse cross-scale attention (SparVAR's CSLA / CS4A hot path) for
AMD Instinct MI355X (gfx950).

The computation runs in libvarsparse.so (HIP kernels behind the C ABI of
include/varsparse.h); this package only marshals arguments.  Importing it
fails if the library has not been built.
"""
from ._lib import (  # noqa: F401
    BF16,
    EHIP,
    EINVAL,
    EUNSUPPORTED,
    FP32,
    LIB_PATH,
    OK,
    VarsparseError,
    attn_fwd,
    attn_fwd_multi,
    attn_fwd_ocache,
    attn_fwd_pair,
    attn_fwd_token,
    build_mask,
    dense_attn_fwd,
    dense_attn_fwd_multi,
    geom_counts,
    join_lists,
    lib,
    make_geom,
    map_indices,
    map_indices_multi,
    ocache_correct,
    window_radius,
)

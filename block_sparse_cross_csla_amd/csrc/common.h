// Internal definitions shared by the varsparse HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "varsparse.h"

namespace vs {

constexpr int kMaxScales = VARSPARSE_MAX_SCALES;

// Geometry of the cache of one query scale, passed by value to kernels.
// Key tiles of scale s have ids tile_base[s] .. tile_base[s+1]-1 (raster within
// the scale); its tokens start at tok_off[s] in the concatenated cache.
struct DevGeom {
    int32_t n_scales;               // scales present in the cache (query scale + 1)
    int32_t tile;
    int32_t side[kMaxScales];
    int32_t nb[kMaxScales];         // tiles per side
    int32_t tile_base[kMaxScales + 1];
    int32_t tok_off[kMaxScales + 1];
};

// Host: fill DevGeom for scales 0..last from a validated varsparse_geom.
inline DevGeom make_dev_geom(const varsparse_geom& g, int last) {
    DevGeom d{};
    d.n_scales = last + 1;
    d.tile = g.tile;
    d.tile_base[0] = 0;
    d.tok_off[0] = 0;
    for (int s = 0; s <= last; ++s) {
        d.side[s] = g.side[s];
        d.nb[s] = (g.side[s] + g.tile - 1) / g.tile;
        d.tile_base[s + 1] = d.tile_base[s] + d.nb[s] * d.nb[s];
        d.tok_off[s + 1] = d.tok_off[s] + g.side[s] * g.side[s];
    }
    return d;
}

// Scale holding key tile `id` (ids are below tile_base[n_scales]).
__device__ __forceinline__ int scale_of_tile(const DevGeom& g, int id) {
    int s = 0;
    while (s + 1 < g.n_scales && id >= g.tile_base[s + 1]) ++s;
    return s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// XCD-aware block order: the hardware deals consecutive workgroup ids round
// robin over the 8 XCDs; remap so that each XCD gets a contiguous range of work
// items (neighbouring query tiles of the same head share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int xcd = bid % kXcd, slot = bid / kXcd;
    const int per = nblocks / kXcd, rem = nblocks % kXcd;
    const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return start + slot;
}

// 16-byte-unit XOR swizzle of LDS key rows: rows 0..15 land on 16 distinct
// units (MFMA A-operand reads of K) and any 4 consecutive rows on distinct
// 4-unit groups (transposed reads of V).  CH = 16-byte units per row.
template <int CH>
__device__ __forceinline__ int swz(int row) {
    return ((row & 3) << (CH == 16 ? 2 : 1)) | ((row >> 2) & (CH == 16 ? 3 : 1));
}

__device__ __forceinline__ void wait_vmcnt(int n) {
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14];
    // expcnt/lgkmcnt at their maximum = do not wait on them.
    if (n == 2) __builtin_amdgcn_s_waitcnt(0x0F72);
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else if (n == 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else __builtin_amdgcn_s_waitcnt(0x0F70);   // anything else: wait for everything
}

// Workgroup barrier with no memory fence: the caller orders its own LDS-DMA
// completions with wait_vmcnt; the asm memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's bytes land at lds + 16 i.  Written as asm
// so that the compiler neither reorders it across the explicit waits and
// barriers of the pipeline nor inserts waits of its own for it; completion is
// tracked by the caller with wait_vmcnt.  There is no destination register.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gaddr), "s"(lds) : "memory", "m0");
}

// Same, addressed as a wave-uniform 64-bit base (SGPR pair) plus a per-lane
// 32-bit byte offset: no 64-bit address arithmetic in VGPRs.
__device__ __forceinline__ void lds_dma16_off(const void* base, int32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)((const __attribute__((address_space(3))) char*)p);
}

}  // namespace vs

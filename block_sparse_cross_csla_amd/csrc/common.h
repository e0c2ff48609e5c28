// Internal definitions shared by the varsparse HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "varsparse.h"

namespace vs {

// Host: let `Kernel` launch with up to `bytes` of dynamic LDS on the current
// device.  The attribute belongs to the function on each device and only
// grows, so the runtime is called once per (kernel, device, larger size):
// repeated launches, and launches under stream capture, make no such call.
// A mutex keeps the recorded size equal to the attribute when threads race.
template <auto Kernel>
hipError_t allow_dynamic_lds(size_t bytes) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static size_t granted[kDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < kDevices;
    std::lock_guard<std::mutex> lock(mu);
    if (tracked && granted[dev] >= bytes) return hipSuccess;
    e = hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && tracked) granted[dev] = bytes;
    return e;
}

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

// Workgroup barrier with no memory fence: the caller orders its own LDS-DMA
// completions with wait_vmcnt; the asm memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) char* lds_ptr;

// 16 bytes per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's bytes land at dst + 16 i (dst wave
// uniform).  The source is a wave-uniform 64-bit base (SGPR pair) plus a
// per-lane 32-bit byte offset: one VALU add per load.  The LDS address goes to
// the instruction through M0, passed as an input operand of the asm, so the
// compiler writes M0 itself and knows it is read (nothing is clobbered); the
// leading s_nop covers the M0-write-to-use hazard, which the compiler cannot
// see inside the asm.  Written as asm so that the compiler does not treat it
// as an LDS store: it would otherwise wait for every outstanding load before
// each later LDS read.  Completion is ordered by the caller with wait_vm /
// wait_all before the workgroup barrier that publishes the bytes.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, lds_ptr dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Same, from a per-lane 64-bit address.
__device__ __forceinline__ void dma16_ptr(const void* gaddr, lds_ptr dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "{m0}"(lds) : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (asm with a memory clobber, so that no load is moved across it).
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_vmcnt(int n) {
    if (n == 2) wait_vm<2>();
    else if (n == 4) wait_vm<4>();
    else if (n == 8) wait_vm<8>();
    else wait_vm<0>();   // anything else: wait for everything
}

// Wait for every outstanding vector-memory and LDS operation of this wave.
__device__ __forceinline__ void wait_all() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

}  // namespace vs

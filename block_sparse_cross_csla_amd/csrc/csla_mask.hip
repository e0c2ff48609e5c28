// CSLA block mask -> per-query-tile kept-tile lists.
//
// SparVAR, ai.info summary, "Methodology in Plain English" (second module):
// project each query of the high-resolution scale onto every earlier scale's
// grid, keep keys inside a per-scale window around the projection, keep the
// sink scales whole, aggregate the token mask into blocks.
//
// The kernel never forms the token mask.  For a t x t query tile the
// projected rows floor(y h / H), y in the tile, form one interval of
// consecutive rows (h <= H, so the projection moves by at most one row per
// query row), likewise the columns; a key tile then holds a kept token pair iff
// the gaps between those intervals and its own row and column ranges are both
// within the radius.  Budget mode ranks tiles by (not sink, admission radius,
// -scale, id), the admission radius being that same gap.
//
// One workgroup (256 threads) per query tile; ascending compaction by a
// workgroup-wide ballot scan.  Integer arithmetic only: bit-exact.
#include "kernel_args.h"

namespace vs {

// Gap between the projected query rows of query-tile row qi and the rows of
// key-tile row ka of a scale of side h (0 if they overlap).  The geometry
// keeps the total token count below 2^30, so every side is below 2^15 and
// (qi t + t - 1) h < H h < 2^30: the products and quotients are exact in 32
// bits (unsigned division, far cheaper than 64-bit division on the GPU).
__device__ __forceinline__ int row_gap(int qi, int ka, int t, int h, int H) {
    const int lo = (int)((uint32_t)(qi * t) * (uint32_t)h / (uint32_t)H);
    const int hi = (int)((uint32_t)(qi * t + t - 1) * (uint32_t)h / (uint32_t)H);
    const int klo = ka * t, khi = min(ka * t + t, h) - 1;
    return max(0, max(klo - hi, lo - khi));
}

__device__ __forceinline__ int tile_gap(const DevGeom& g, int s, int local, int ti, int tj, int H) {
    const int nb = g.nb[s], t = g.tile, h = g.side[s];
    const int a = local / nb, b = local - a * nb;
    return max(row_gap(ti, a, t, h, H), row_gap(tj, b, t, h, H));
}

__global__ __launch_bounds__(256) void csla_mask_kernel(const MaskArgs a) {
    extern __shared__ uint64_t rank_key[];   // budget mode: one packed key per tile
    __shared__ int wave_cnt[4];
    const int qt = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.g.side[a.q_scale];
    const int nbq = a.g.nb[a.q_scale];
    const int ti = qt / nbq, tj = qt - ti * nbq;
    const int nkb = a.nkb;
    const bool budget = a.budget > 0;

    if (budget) {
        for (int j = tid; j < nkb; j += 256) {
            const int s = scale_of_tile(a.g, j);
            const uint64_t dist = (uint64_t)tile_gap(a.g, s, j - a.g.tile_base[s], ti, tj, H);
            rank_key[j] = ((uint64_t)(s >= a.n_sink) << 62) | (dist << 30) |
                          ((uint64_t)(31 - s) << 25) | (uint64_t)j;
        }
        __syncthreads();
    }

    int base = 0;
    for (int c0 = 0; c0 < nkb; c0 += 256) {
        const int j = c0 + tid;
        bool keep = false;
        if (j < nkb) {
            if (budget) {
                const uint64_t mine = rank_key[j];
                int rank = 0;
                for (int i = 0; i < nkb; ++i) rank += rank_key[i] < mine;
                keep = rank < a.keep_n;
            } else {
                const int s = scale_of_tile(a.g, j);
                keep = s < a.n_sink ||
                       (a.radius[s] >= 0 && tile_gap(a.g, s, j - a.g.tile_base[s], ti, tj, H) <= a.radius[s]);
            }
            if (a.mask != nullptr) a.mask[(int64_t)qt * nkb + j] = keep ? 1 : 0;
        }
        const uint64_t bal = __ballot(keep);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = base, total = 0;
        for (int w = 0; w < 4; ++w) {
            if (w < wave) before += wave_cnt[w];
            total += wave_cnt[w];
        }
        if (keep) a.kv_idx[(int64_t)qt * nkb + before + __popcll(bal & ((1ull << lane) - 1))] = j;
        __syncthreads();
        base += total;
    }
    for (int j = base + tid; j < nkb; j += 256) a.kv_idx[(int64_t)qt * nkb + j] = -1;
    if (tid == 0) a.kv_cnt[qt] = base;
}

hipError_t launch_csla_mask(const MaskArgs& a, int nqb, hipStream_t stream) {
    const size_t shmem = a.budget > 0 ? (size_t)a.nkb * sizeof(uint64_t) : 0;
    hipLaunchKernelGGL(csla_mask_kernel, dim3(nqb), dim3(256), shmem, stream, a);
    return hipGetLastError();
}

}  // namespace vs

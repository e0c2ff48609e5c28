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

__device__ __forceinline__ int tile_gap(int nb, int t, int h, int local, int ti, int tj, int H) {
    const int a = local / nb, b = local - a * nb;
    return max(row_gap(ti, a, t, h, H), row_gap(tj, b, t, h, H));
}

// The geometry of scale `lane` held in that lane (every wave alike), so that
// a thread finds the scale of its key tile, and that scale's numbers, with a
// uniform loop of lane reads (readlane ignores the execution mask, so this
// also holds in divergent code), not with a chain of dependent loads from the
// kernel arguments.
struct ScaleOf {
    int s, tb, nb, side, radius;
};

struct LaneScales {
    int tb, nb, side, radius;   // tile_base / nb / side / radius of scale `lane`
    int n;                      // number of scales

    __device__ static LaneScales load(const MaskArgs& a, int lane) {
        LaneScales r;
        r.n = a.g.n_scales;
        const bool in = lane < r.n;
        const int s = min(lane, kMaxScales - 1);
        r.tb = in ? a.g.tile_base[s] : 0;
        r.nb = in ? a.g.nb[s] : 1;
        r.side = in ? a.g.side[s] : 1;
        r.radius = in ? a.radius[s] : -1;
        return r;
    }
    // key tile `id` lies in the last scale that starts at or before it
    __device__ ScaleOf find(int id) const {
        ScaleOf r{0, __builtin_amdgcn_readlane(tb, 0), __builtin_amdgcn_readlane(nb, 0),
                  __builtin_amdgcn_readlane(side, 0), __builtin_amdgcn_readlane(radius, 0)};
        for (int u = 1; u < n; ++u) {
            const int b = __builtin_amdgcn_readlane(tb, u);
            if (id >= b) {
                r.s = u;
                r.tb = b;
                r.nb = __builtin_amdgcn_readlane(nb, u);
                r.side = __builtin_amdgcn_readlane(side, u);
                r.radius = __builtin_amdgcn_readlane(radius, u);
            }
        }
        return r;
    }
};

__global__ __launch_bounds__(256) void csla_mask_kernel(const MaskArgs a) {
    extern __shared__ uint64_t rank_key[];   // budget mode: one packed key per tile
    __shared__ int wave_cnt[4];
    const int qt = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.g.side[a.q_scale];
    const int nbq = a.g.nb[a.q_scale];
    const int ti = qt / nbq, tj = qt - ti * nbq;
    const int nkb = a.nkb;
    const bool budget = a.budget > 0;
    const LaneScales ls = LaneScales::load(a, lane);
    auto gap = [&](int j, const ScaleOf& f) { return tile_gap(f.nb, a.g.tile, f.side, j - f.tb, ti, tj, H); };

    if (budget) {
        for (int j = tid; j < nkb; j += 256) {
            const ScaleOf f = ls.find(j);
            const int s = f.s;
            const uint64_t dist = (uint64_t)gap(j, f);
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
                const ScaleOf f = ls.find(j);
                keep = f.s < a.n_sink || (f.radius >= 0 && gap(j, f) <= f.radius);
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

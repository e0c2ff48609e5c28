// Join of two kept-tile lists per query tile: union or intersection of the
// CS4A-mapped tiles and the CSLA window tiles of the same query scale
// (SparVAR, ai.info summary, "Main Findings": the two modules are used
// together on the last scales, CSLA with windows 3/5/7; "Methodology in Plain
// English": CSLA's mask does not depend on the decision scale, so the two
// tile sets are built apart and joined here).
//
// Integer only.  One wave per list row, its own bitmap of nkb bits in LDS:
// union sets the bits of both lists and emits the set bits in ascending order
// (32 tiles per lane per step, wave prefix sum of popcounts); intersection
// sets the bits of list b and keeps, in order, the entries of list a whose
// bit is set (ballot compaction).  Entries outside [0, nkb) are ignored and
// counts are clamped to [0, nkb], so a malformed list cannot move an access
// out of bounds.  The row is padded with -1 up to nkb entries.
#include "kernel_args.h"

namespace vs {

constexpr int kJoinWaves = 4;

__device__ __forceinline__ int wave_prefix_excl(int v, int lane, int* total) {
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    *total = __shfl(x, 63, 64);
    return x - v;
}

__global__ __launch_bounds__(256) void join_lists_kernel(const JoinArgs a) {
    extern __shared__ uint32_t join_bits[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kJoinWaves + wave;
    const bool valid = row < (int64_t)a.sets * a.rows;
    uint32_t* bm = join_bits + wave * a.words;

    int set = 0, r = 0;
    if (valid) { set = (int)(row / a.rows); r = (int)(row - (int64_t)set * a.rows); }
    const int64_t ra = (int64_t)(a.a_per_set ? set : 0) * a.rows + r;
    const int64_t rb = (int64_t)(a.b_per_set ? set : 0) * a.rows + r;
    const int32_t* ai = a.a_idx + ra * a.nkb;
    const int32_t* bi = a.b_idx + rb * a.nkb;
    const int na = valid ? min(max(a.a_cnt[ra], 0), a.nkb) : 0;
    const int nb = valid ? min(max(a.b_cnt[rb], 0), a.nkb) : 0;

    for (int w = lane; w < a.words; w += 64) bm[w] = 0u;
    __syncthreads();
    if (a.join == VARSPARSE_JOIN_UNION) {
        for (int i = lane; i < na; i += 64) {
            const int id = ai[i];
            if (id >= 0 && id < a.nkb) atomicOr(&bm[id >> 5], 1u << (id & 31));
        }
    }
    for (int i = lane; i < nb; i += 64) {
        const int id = bi[i];
        if (id >= 0 && id < a.nkb) atomicOr(&bm[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    if (!valid) return;

    int32_t* out = a.out_idx + row * a.nkb;
    int n = 0;
    if (a.join == VARSPARSE_JOIN_UNION) {
        for (int w0 = 0; w0 < a.words; w0 += 64) {
            const int w = w0 + lane;
            uint32_t word = w < a.words ? bm[w] : 0u;
            int total;
            int pos = n + wave_prefix_excl(__popc(word), lane, &total);
            while (word) {
                const int bit = __ffs(word) - 1;
                out[pos++] = w * 32 + bit;
                word &= word - 1;
            }
            n += total;
        }
    } else {
        for (int i0 = 0; i0 < na; i0 += 64) {
            const int i = i0 + lane;
            const int id = i < na ? ai[i] : -1;
            const bool keep = id >= 0 && id < a.nkb && ((bm[id >> 5] >> (id & 31)) & 1u);
            const uint64_t m = __ballot(keep);
            if (keep) out[n + __popcll(m & ((1ull << lane) - 1ull))] = id;
            n += __popcll(m);
        }
    }
    for (int i = n + lane; i < a.nkb; i += 64) out[i] = -1;
    if (lane == 0) a.out_cnt[row] = n;
}

hipError_t launch_join_lists(const JoinArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.sets * a.rows;
    dim3 grid((unsigned)((rows + kJoinWaves - 1) / kJoinWaves)), block(64 * kJoinWaves);
    const size_t lds = (size_t)kJoinWaves * a.words * sizeof(uint32_t);
    hipLaunchKernelGGL(join_lists_kernel, grid, block, lds, stream, a);
    return hipGetLastError();
}

}  // namespace vs

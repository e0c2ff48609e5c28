// CS4A: decision-scale block scores, top-p selection and cross-scale index
// mapping (SparVAR, ai.info summary, "Methodology in Plain English", first
// module; "Main Findings", the decision scale).
//
// cs4a_score_kernel: full attention of the decision scale's queries over the
// keys of scales 0..D, reduced to one number per (query tile, key tile): the
// mean over the tile's queries of the softmax mass falling in the key tile.
// Single pass: per key tile, partial sums of exp2(s*c - m) relative to the
// query's running max m (raised lazily, the partials rescaled when it is);
// the row total is the sum of the partials.  The key tiles are split between
// four wave pairs (tiles equal mod 4) whose maxima and sums are merged
// exactly at the end.  QK^T runs on bf16 MFMA (32x32x16) with K staged in
// LDS ahead of use.  Reductions run in a fixed order: scores are
// bit-reproducible.
//
// cs4a_select_map_kernel: one wave per (batch, head, target scale, target
// query tile); one launch maps the selection onto up to kMaxTargets scales.
// Top-p (or Top-K) on integer-quantised scores (exact, associative) of the
// parent decision tile, kept as a bitset in registers, then the target-scale lists: parent tile by floor scaling, tiles below the
// decision scale copied, decision-scale tiles expanded to their footprint on
// every scale from D to the target, sink tiles added.
#include "kernel_args.h"

namespace vs {

constexpr int kScoreParts = 4;                          // key-tile parts
constexpr int kScoreStages = 2;                         // LDS ring depth per part
constexpr int kScoreThreads = 2 * 64 * kScoreParts;     // two query halves per part

// One chunk of the key walk: up to 4 rows x 8 columns of one key tile.
struct ScoreChunk {
    int32_t base;       // token of the first key
    int32_t stride;     // tokens per row of its scale
    int32_t tile;       // key-tile id
    int32_t shape;      // rows | cols << 4
};

// Maximum of this lane's 16 scores of a chunk (a pairwise tree: fmax is
// exact, so the order only shortens the dependency chain).
__device__ __forceinline__ float chunk_max(const f32x16& s) {
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(s[i], s[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], m[i + 4]);
    return fmaxf(fmaxf(m[0], m[2]), fmaxf(m[1], m[3]));
}

// Sum of exp2(s c - m) over this lane's 16 scores of a chunk, in a fixed
// pairwise order.
__device__ __forceinline__ float chunk_sumexp(const f32x16& s, float c, float m) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = p[2 * i] + p[2 * i + 1];
    return (p[0] + p[1]) + (p[2] + p[3]);
}

// Score of one (query tile, key tile): the mean over the tile's 64 queries of
// acc[q] f[q] (a query's partial sum and its normalising factor), summed by
// a group of 8 consecutive lanes in a fixed order (8 values per lane, then a
// butterfly over the group; every lane of the group ends with the total).
__device__ __forceinline__ float tile_mean64(const float* acc, const float* f, int lane8) {
#pragma clang fp contract(off)
    const float4 a0 = *(const float4*)(acc + 8 * lane8), a1 = *(const float4*)(acc + 8 * lane8 + 4);
    const float4 f0 = *(const float4*)(f + 8 * lane8), f1 = *(const float4*)(f + 8 * lane8 + 4);
    float x = ((a0.x * f0.x + a0.y * f0.y) + (a0.z * f0.z + a0.w * f0.w)) +
              ((a1.x * f1.x + a1.y * f1.y) + (a1.z * f1.z + a1.w * f1.w));
    x += __shfl_xor(x, 1, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 4, 8);
    return x * (1.0f / 64.0f);
}

// Eight waves per decision query tile: wave w takes query rows
// 4 (w & 1) .. 4 (w & 1) + 3 (32 queries) and the key tiles of part w >> 1
// (tiles part, part + 4, ...).  The chunk table (every key tile split in
// halves of up to 4 rows) is built once per workgroup in LDS, one thread per
// key tile and a per-part prefix sum, so the walk costs one LDS broadcast
// read per chunk.  The two waves of a part share its K chunks, loaded
// HBM -> LDS with global_load_lds (16 B per lane, whole rows per
// instruction) into a ring of kScoreStages buffers, kScoreStages - 1 chunks
// ahead of use, one workgroup barrier per step; two workgroups share a CU.
// Single pass: each lane keeps, per key tile of its part, the partial sum
// of exp2(s c - m) over its query's keys relative to its running max m
// (raised lazily, the partials rescaled when it is); at the end the parts'
// maxima and sums are merged exactly, every partial is normalised by its
// query's total, and each key tile's score is summed over its 64 queries in
// a fixed order (bit-reproducible).
template <int D>
__global__ __launch_bounds__(kScoreThreads) void cs4a_score_kernel(const ScoreArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int STAGE = 32 * ROWB;
    constexpr int RPL = 1024 / ROWB;
    constexpr int LOADS = 16 / RPL;                                // load instructions per wave per chunk
    constexpr int NST = kScoreStages;
    constexpr float kLazy = 8.0f;
    extern __shared__ __attribute__((aligned(1024))) char dyn[];
    char* kst_base = dyn;                                          // [part][stage][STAGE]
    const int tpp = a.nkb / 2 + 2;                                 // table entries per part (>= 2 ceil(nkb / 4))
    ScoreChunk* table = (ScoreChunk*)(dyn + kScoreParts * NST * STAGE);   // [part][tpp]
    int* halves = (int*)(table + kScoreParts * tpp);                         // [nkb]
    int* nchunks = halves + a.nkb;                                 // [part]
    // 16-byte aligned from here on: the tile sums read acc and mrow as float4
    float* mrow = (float*)(dyn + ((((char*)(nchunks + kScoreParts) - dyn) + 15) & ~15));   // [part][64]
    float* lrow = mrow + 64 * kScoreParts;                         // [part][64]
    float* acc = lrow + 64 * kScoreParts;                                       // [nkb][64 queries]

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qh = wave & 1, par = wave >> 1;
    const int n = lane & 31, g = lane >> 5;
    const int q = qh * 32 + n;                                     // query within the tile
    const int bh = blockIdx.x / a.nqb, qt = blockIdx.x - bh * a.nqb;
    const int b = bh / a.H, h = bh - b * a.H;
    const int nkb = a.nkb;

    const int nbq = a.d_side >> 3;
    const int ti = qt / nbq, tj = qt - ti * nbq;
    const int64_t tok = (int64_t)(8 * ti + 4 * qh + (n >> 3)) * a.d_side + 8 * tj + (n & 7);
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;

    // chunk table: one thread per key tile
    int my_tile_rows = 0, my_s = 0, my_ta = 0, my_tb = 0;
    if (tid < nkb) {
        my_s = scale_of_tile(a.g, tid);
        const int local = tid - a.g.tile_base[my_s];
        my_ta = local / a.g.nb[my_s];
        my_tb = local - my_ta * a.g.nb[my_s];
        my_tile_rows = min(8, a.g.side[my_s] - 8 * my_ta);
        halves[tid] = my_tile_rows > 4 ? 2 : 1;
    }
    if (tid < kScoreParts) nchunks[tid] = 0;
    for (int i = tid; i < nkb * 64; i += kScoreThreads) acc[i] = 0.0f;
    __syncthreads();
    if (tid < nkb) {
        const int p = tid % kScoreParts;
        int off = 0;
        for (int j = p; j < tid; j += kScoreParts) off += halves[j];
        const int side = a.g.side[my_s];
        const int cols = min(8, side - 8 * my_tb);
        for (int hh = 0; hh < halves[tid]; ++hh) {
            ScoreChunk c;
            c.base = a.g.tok_off[my_s] + (8 * my_ta + 4 * hh) * side + 8 * my_tb;
            c.stride = side;
            c.tile = tid;
            c.shape = min(4, my_tile_rows - 4 * hh) | (cols << 4);
            table[p * tpp + off + hh] = c;
        }
        if (tid + kScoreParts >= nkb) nchunks[p] = off + halves[tid];   // last tile of its part
    }
    __syncthreads();
    const int nch = nchunks[par];
    int nmax = 0;
#pragma unroll
    for (int p = 0; p < kScoreParts; ++p) nmax = max(nmax, nchunks[p]);
    const ScoreChunk* mytab = table + par * tpp;
    wait_vmcnt(0);   // Q is in registers before LDS-DMA traffic starts
    // ... and the compiler is told so (an empty asm that reads and rewrites
    // the operands): otherwise its own waits for the Q loads stay in front of
    // the MFMAs of every chunk, where a vmcnt wait also waits for the chunk
    // loads running ahead (asm, which it does not count)
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(qreg[s]));

    const lds_ptr kst0 = (lds_ptr)kst_base + par * NST * STAGE;
    auto issue = [&](int ci) {
        const ScoreChunk c = mytab[ci];
        const int nrows = c.shape & 15, ncols = c.shape >> 4;
        const lds_ptr kst = kst0 + (ci % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int row = 16 * qh + i * RPL + lane / CH;
            const int lc = (lane % CH) ^ swz<CH>(row);
            const int r = row >> 3, col = row & 7;
            const bool valid = r < nrows && col < ncols;
            const int t = valid ? c.base + r * c.stride + col : c.base;
            dma16_ptr(kh + t * a.sk_t + lc * 8, kst + (16 * qh + i * RPL) * ROWB);
        }
    };

    const float cl = a.scale_log2;
    float m_run = -INFINITY;
    for (int k = 0; k < NST - 1 && k < nch; ++k) issue(k);
    for (int ci = 0; ci < nmax; ++ci) {
        const int ahead = min(NST - 2, nch - 1 - ci);             // chunks issued after chunk ci
        if (ahead >= 2) wait_vmcnt(2 * LOADS);
        else if (ahead == 1) wait_vmcnt(LOADS);
        else wait_vmcnt(0);
        wg_barrier();
        if (ci + NST - 1 < nch) issue(ci + NST - 1);
        if (ci < nch) {
            const ScoreChunk c = mytab[ci];
            const int cr = c.shape & 15, ccn = c.shape >> 4, ct = c.tile;
            const char* kst = kst_base + (par * NST + ci % NST) * STAGE;
            f32x16 sacc = (f32x16)0.0f;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int pc = (2 * s + g) ^ swz<CH>(n);
                const bf16x8 kop = *(const bf16x8*)(kst + n * ROWB + pc * 16);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[s], sacc, 0, 0, 0);
            }
            if (cr < 4 || ccn < 8) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = i >> 2, col = 4 * g + (i & 3);
                    if (!(r < cr && col < ccn)) sacc[i] = -INFINITY;
                }
            }
            float mx = chunk_max(sacc);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float cand = mx * cl;
            const bool need = cand > m_run + kLazy;
            if (__ballot(need)) {
                if (need) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - cand);
                    if (g == 0)
                        for (int kt = par; kt <= ct; kt += kScoreParts) acc[kt * 64 + q] *= alpha;
                    m_run = cand;
                }
            }
            float part = chunk_sumexp(sacc, cl, m_run);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
            part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // both halves of the query's keys
            if (g == 0) acc[ct * 64 + q] += part;
        }
    }

    // merge the parts: common max M, total l, then each (part, query)'s
    // normalising factor
    float l_mine = 0.0f, fq = 0.0f;
    if (g == 0)
        for (int kt = par; kt < nkb; kt += kScoreParts) l_mine += acc[kt * 64 + q];
    if (g == 0) {
        mrow[par * 64 + q] = m_run;
        lrow[par * 64 + q] = l_mine;
    }
    __syncthreads();
    if (g == 0) {
        float M = mrow[q];
#pragma unroll
        for (int p = 1; p < kScoreParts; ++p) M = fmaxf(M, mrow[p * 64 + q]);
        float l_q = 0.0f;
#pragma unroll
        for (int p = 0; p < kScoreParts; ++p) {
            const float mp = mrow[p * 64 + q];
            if (mp != -INFINITY) l_q += lrow[p * 64 + q] * __builtin_amdgcn_exp2f(mp - M);
        }
        fq = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M) / l_q;
    }
    __syncthreads();   // every part's maximum and sum read
    if (g == 0) mrow[par * 64 + q] = fq;   // now: the normalising factor of (part, query)
    __syncthreads();
    float* out = a.scores + ((int64_t)bh * a.nqb + qt) * nkb;
    for (int kt = tid >> 3; kt < nkb; kt += kScoreThreads / 8) {
        const float v = tile_mean64(acc + kt * 64, mrow + (kt % kScoreParts) * 64, tid & 7);
        if ((tid & 7) == 0) out[kt] = v;
    }
}

// Two decision query tiles per workgroup (16 waves): wave w takes query half
// w & 1 of tile (w >> 1) & 1 and the key tiles of part w >> 2.  The four
// waves of a part share its K chunks (each loads 8 of the 32 rows), so each
// chunk in LDS serves 128 queries: half the K loads per query of the
// one-tile form, and room in LDS for an NST-deep ring at 16 waves per CU
// (the one-tile form runs two workgroups of 8 waves per CU with a 2-deep
// ring: its waves wait on their next chunk).  Per query the arithmetic and
// its order are those of cs4a_score_kernel: the scores are bit-identical.
constexpr int kScore2Tiles = 2;
constexpr int kScore2Threads = 2 * 64 * kScoreParts * kScore2Tiles;

template <int D, int NST>
__global__ __launch_bounds__(kScore2Threads) void cs4a_score2_kernel(const ScoreArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int STAGE = 32 * ROWB;
    constexpr int RPL = 1024 / ROWB;
    constexpr int LOADS = 8 / RPL;                                 // load instructions per wave per chunk
    constexpr int NQ = 64 * kScore2Tiles;                          // queries per workgroup
    constexpr float kLazy = 8.0f;
    extern __shared__ __attribute__((aligned(1024))) char dyn[];
    char* kst_base = dyn;                                          // [part][stage][STAGE]
    const int tpp = a.nkb / 2 + 2;
    ScoreChunk* table = (ScoreChunk*)(dyn + kScoreParts * NST * STAGE);   // [part][tpp]
    int* halves = (int*)(table + kScoreParts * tpp);                         // [nkb]
    int* nchunks = halves + a.nkb;                                 // [part]
    // 16-byte aligned from here on: the tile sums read acc and mrow as float4
    float* mrow = (float*)(dyn + ((((char*)(nchunks + kScoreParts) - dyn) + 15) & ~15));   // [part][NQ]
    float* lrow = mrow + NQ * kScoreParts;                         // [part][NQ]
    float* acc = lrow + NQ * kScoreParts;                          // [nkb][NQ]

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qh = wave & 1, tq = (wave >> 1) & 1, par = wave >> 2;
    const int wip = wave & 3;                                      // wave within its part
    const int n = lane & 31, g = lane >> 5;
    const int q = tq * 64 + qh * 32 + n;                           // query within the workgroup
    const int ntp = (a.nqb + 1) >> 1;
    const int bh = blockIdx.x / ntp, tp = blockIdx.x - bh * ntp;
    const int qt = 2 * tp + tq;
    const bool tile_ok = qt < a.nqb;                               // an odd last tile pairs with nothing
    const int b = bh / a.H, h = bh - b * a.H;
    const int nkb = a.nkb;

    const int nbq = a.d_side >> 3;
    const int qtc = tile_ok ? qt : a.nqb - 1;
    const int ti = qtc / nbq, tj = qtc - ti * nbq;
    const int64_t tok = (int64_t)(8 * ti + 4 * qh + (n >> 3)) * a.d_side + 8 * tj + (n & 7);
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;

    // chunk table: one thread per key tile
    int my_tile_rows = 0, my_s = 0, my_ta = 0, my_tb = 0;
    if (tid < nkb) {
        my_s = scale_of_tile(a.g, tid);
        const int local = tid - a.g.tile_base[my_s];
        my_ta = local / a.g.nb[my_s];
        my_tb = local - my_ta * a.g.nb[my_s];
        my_tile_rows = min(8, a.g.side[my_s] - 8 * my_ta);
        halves[tid] = my_tile_rows > 4 ? 2 : 1;
    }
    if (tid < kScoreParts) nchunks[tid] = 0;
    for (int i = tid; i < nkb * NQ; i += kScore2Threads) acc[i] = 0.0f;
    __syncthreads();
    if (tid < nkb) {
        const int p = tid % kScoreParts;
        int off = 0;
        for (int j = p; j < tid; j += kScoreParts) off += halves[j];
        const int side = a.g.side[my_s];
        const int cols = min(8, side - 8 * my_tb);
        for (int hh = 0; hh < halves[tid]; ++hh) {
            ScoreChunk c;
            c.base = a.g.tok_off[my_s] + (8 * my_ta + 4 * hh) * side + 8 * my_tb;
            c.stride = side;
            c.tile = tid;
            c.shape = min(4, my_tile_rows - 4 * hh) | (cols << 4);
            table[p * tpp + off + hh] = c;
        }
        if (tid + kScoreParts >= nkb) nchunks[p] = off + halves[tid];
    }
    __syncthreads();
    const int nch = nchunks[par];
    int nmax = 0;
#pragma unroll
    for (int p = 0; p < kScoreParts; ++p) nmax = max(nmax, nchunks[p]);
    const ScoreChunk* mytab = table + par * tpp;
    wait_vmcnt(0);   // Q is in registers before LDS-DMA traffic starts
    // ... and the compiler is told so (an empty asm that reads and rewrites
    // the operands): otherwise its own waits for the Q loads stay in front of
    // the MFMAs of every chunk, where a vmcnt wait also waits for the chunk
    // loads running ahead (asm, which it does not count)
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(qreg[s]));

    const lds_ptr kst0 = (lds_ptr)kst_base + par * NST * STAGE;
    auto issue = [&](int ci) {
        const ScoreChunk c = mytab[ci];
        const int nrows = c.shape & 15, ncols = c.shape >> 4;
        const lds_ptr kst = kst0 + (ci % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int row = 8 * wip + i * RPL + lane / CH;
            const int lc = (lane % CH) ^ swz<CH>(row);
            const int r = row >> 3, col = row & 7;
            const bool valid = r < nrows && col < ncols;
            const int t = valid ? c.base + r * c.stride + col : c.base;
            dma16_ptr(kh + t * a.sk_t + lc * 8, kst + (8 * wip + i * RPL) * ROWB);
        }
    };

    const float cl = a.scale_log2;
    float m_run = -INFINITY;
    for (int k = 0; k < NST - 1 && k < nch; ++k) issue(k);
    for (int ci = 0; ci < nmax; ++ci) {
        const int ahead = min(NST - 2, nch - 1 - ci);             // chunks issued after chunk ci
        if (ahead >= 2) wait_vmcnt(2 * LOADS);
        else if (ahead == 1) wait_vmcnt(LOADS);
        else wait_vmcnt(0);
        wg_barrier();
        if (ci + NST - 1 < nch) issue(ci + NST - 1);
        if (ci < nch) {
            const ScoreChunk c = mytab[ci];
            const int cr = c.shape & 15, ccn = c.shape >> 4, ct = c.tile;
            const char* kst = kst_base + (par * NST + ci % NST) * STAGE;
            f32x16 sacc = (f32x16)0.0f;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int pc = (2 * s + g) ^ swz<CH>(n);
                const bf16x8 kop = *(const bf16x8*)(kst + n * ROWB + pc * 16);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[s], sacc, 0, 0, 0);
            }
            if (cr < 4 || ccn < 8) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = i >> 2, col = 4 * g + (i & 3);
                    if (!(r < cr && col < ccn)) sacc[i] = -INFINITY;
                }
            }
            float mx = chunk_max(sacc);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float cand = mx * cl;
            const bool need = cand > m_run + kLazy;
            if (__ballot(need)) {
                if (need) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - cand);
                    if (g == 0)
                        for (int kt = par; kt <= ct; kt += kScoreParts) acc[kt * NQ + q] *= alpha;
                    m_run = cand;
                }
            }
            float part = chunk_sumexp(sacc, cl, m_run);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
            part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (g == 0) acc[ct * NQ + q] += part;
        }
    }

    // merge the parts: common max M, total l, then each (part, query)'s
    // normalising factor
    float l_mine = 0.0f, fq = 0.0f;
    if (g == 0)
        for (int kt = par; kt < nkb; kt += kScoreParts) l_mine += acc[kt * NQ + q];
    if (g == 0) {
        mrow[par * NQ + q] = m_run;
        lrow[par * NQ + q] = l_mine;
    }
    __syncthreads();
    if (g == 0) {
        float M = mrow[q];
#pragma unroll
        for (int p = 1; p < kScoreParts; ++p) M = fmaxf(M, mrow[p * NQ + q]);
        float l_q = 0.0f;
#pragma unroll
        for (int p = 0; p < kScoreParts; ++p) {
            const float mp = mrow[p * NQ + q];
            if (mp != -INFINITY) l_q += lrow[p * NQ + q] * __builtin_amdgcn_exp2f(mp - M);
        }
        fq = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M) / l_q;
    }
    __syncthreads();   // every part's maximum and sum read
    if (g == 0) mrow[par * NQ + q] = fq;   // now: the normalising factor of (part, query)
    __syncthreads();
    for (int e = tid >> 3; e < kScore2Tiles * nkb; e += kScore2Threads / 8) {
        const int t2 = e / nkb, kt = e - t2 * nkb;
        if (2 * tp + t2 >= a.nqb) continue;   // the same for the 8 lanes of a group
        const float v = tile_mean64(acc + kt * NQ + t2 * 64, mrow + (kt % kScoreParts) * NQ + t2 * 64, tid & 7);
        if ((tid & 7) == 0) a.scores[((int64_t)bh * a.nqb + 2 * tp + t2) * nkb + kt] = v;
    }
}

__device__ __forceinline__ int64_t quantise(float s) {
    const float x = s * 16777216.0f;   // exact: power-of-two scaling
    return x >= 0.0f ? (int64_t)floorf(x) : 0;
}

// One workgroup = 4 waves = 4 target query tiles of one (batch, head).  Each
// wave selects the key tiles of its parent decision tile (scores staged in
// LDS, one quantised score per entry; ranks and prefix masses by broadcast
// reads), keeps the selection as a bitset in registers (one ballot per 64
// tiles), then decides every target key tile and compacts the list with
// ballots, one key scale at a time: each decision row block's footprint on
// the key scale is computed once per wave (exact integer quotients), and a
// key tile is kept iff a selected decision tile's row and column footprints
// both meet it.  The wave whose target tile is the first child of its parent
// also writes the parent's selection (sel_cnt / sel_idx) when asked to.
__global__ __launch_bounds__(256) void cs4a_select_map_kernel(const SelMapArgs a) {
    __shared__ int64_t mq[4][256];   // quantised scores of each wave's parent tile
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // block -> (b h, target, group of 4 target query tiles)
    const int bh = blockIdx.x / a.groups_total;
    const int gi = blockIdx.x - bh * a.groups_total;
    int tg = 0;
    while (tg + 1 < a.n_targets && a.group_base[tg + 1] <= gi) ++tg;
    const int T = a.t_scale[tg], nqbT = a.nqbT[tg], nkbT = a.nkbT[tg];
    const int qt = (gi - a.group_base[tg]) * 4 + wave;
    if (qt >= nqbT) return;   // whole wave leaves; no workgroup barrier below
    const int nkbD = a.nkbD;
    const int D = a.d_scale, t = a.g.tile;
    const int hD = a.g.side[D], nbD = a.g.nb[D], nbT = a.g.nb[T];
    const int ti = qt / nbT, tj = qt - ti * nbT;
    const int pi = ti * nbD / nbT, pj = tj * nbD / nbT;
    const int parent = pi * nbD + pj;

    // ---- top-p selection of the parent tile
    const float* sc = a.scores + ((int64_t)bh * a.nqbD + parent) * nkbD;
    int64_t tot = 0;
    for (int j = lane; j < nkbD; j += 64) {
        const int64_t m = quantise(sc[j]);
        mq[wave][j] = m;
        tot += m;
    }
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
    const double thr = ceil(a.top_p * (double)tot);
    uint64_t sel[4] = {0, 0, 0, 0};   // bit j of the selection, 64 tiles per word
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        const int j = 64 * w4 + lane;
        bool keep = false;
        if (64 * w4 < nkbD) {
            if (j < nkbD) {
                const int64_t mj = mq[wave][j];
                // mass (top-p) or number (Top-K) of the tiles ordered before j
                const bool by_mass = a.rule == 0;
                int64_t before = 0;
                for (int i = 0; i < nkbD; ++i) {
                    const int64_t mi = mq[wave][i];
                    before += (mi > mj || (mi == mj && i < j)) ? (by_mass ? mi : 1) : 0;
                }
                keep = by_mass ? (double)before < thr : before < a.k_keep;
            }
            sel[w4] = __ballot(keep);
        }
    }
    const bool first_row = ti == 0 || (ti - 1) * nbD / nbT != pi;
    const bool first_col = tj == 0 || (tj - 1) * nbD / nbT != pj;
    if (a.sel_idx != nullptr && tg == 0 && first_row && first_col) {
        int base = 0;
        int32_t* out = a.sel_idx + ((int64_t)bh * a.nqbD + parent) * nkbD;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            const int j = 64 * w4 + lane;
            if ((sel[w4] >> lane) & 1) out[base + __popcll(sel[w4] & ((1ull << lane) - 1))] = j;
            base += __popcll(sel[w4]);
        }
        for (int j = base + lane; j < nkbD; j += 64) out[j] = -1;
        if (lane == 0) a.sel_cnt[(int64_t)bh * a.nqbD + parent] = base;
    }
    auto selected = [&](int id) -> bool {
        const uint64_t word = id < 64 ? sel[0] : id < 128 ? sel[1] : id < 192 ? sel[2] : sel[3];
        return (word >> (id & 63)) & 1;
    };

    // ---- mapping onto the target scale, one key scale at a time (uniform
    // loop, ascending ids).  srows[sa]: bit sb set iff decision tile (sa, sb)
    // is selected; fp[sa]: the rows [lo, hi] of scale s that decision row
    // block sa covers (the same numbers serve columns: grids are square).
    __shared__ uint32_t srows[4][16];
    __shared__ int2 fp[4][16];
    const int tbD = a.g.tile_base[D];
    // the geometry of scale `lane` in that lane (read with readlane below, not
    // through a chain of dependent scalar loads per scale)
    const int g_tb = lane <= a.g.n_scales ? a.g.tile_base[min(lane, kMaxScales)] : 0;
    const int g_side = lane < a.g.n_scales ? a.g.side[min(lane, kMaxScales - 1)] : 0;
    const int g_nb = lane < a.g.n_scales ? a.g.nb[min(lane, kMaxScales - 1)] : 1;
    if (lane < nbD) {
        uint32_t r = 0;
        for (int sb = 0; sb < nbD; ++sb) r |= (uint32_t)selected(tbD + lane * nbD + sb) << sb;
        srows[wave][lane] = r;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's LDS writes before its reads
    int base = 0;
    int32_t* out = a.kv_idx[tg] + ((int64_t)bh * nqbT + qt) * nkbT;
    for (int s = 0; s <= T; ++s) {
        const int tb0 = __builtin_amdgcn_readlane(g_tb, s), tb1 = __builtin_amdgcn_readlane(g_tb, s + 1);
        const int hs = __builtin_amdgcn_readlane(g_side, s), nbs = __builtin_amdgcn_readlane(g_nb, s);
        if (s >= D) {
            if (lane < nbD) {
                // floor / ceil of exact quotients: sides are below 2^15, products below 2^30
                const int ey = min(lane * t + t, hD);
                const int lo = (int)((uint32_t)(lane * t) * (uint32_t)hs / (uint32_t)hD);
                const int hi = (int)(((uint32_t)ey * (uint32_t)hs + (uint32_t)hD - 1u) / (uint32_t)hD) - 1;
                fp[wave][lane] = make_int2(lo, hi);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
        // decision row (or column) blocks whose footprint meets key row block k
        auto cover = [&](int k) -> uint32_t {
            const int klo = k * t, khi = min(k * t + t, hs) - 1;
            uint32_t m = 0;
            for (int sa = 0; sa < nbD; ++sa) {
                const int2 f = fp[wave][sa];
                m |= (uint32_t)(klo <= f.y && f.x <= khi) << sa;
            }
            return m;
        };
        for (int c0 = tb0; c0 < tb1; c0 += 64) {
            const int j = c0 + lane;
            bool keep = false;
            if (j < tb1) {
                if (s < a.n_sink) {
                    keep = true;
                } else if (s < D) {
                    keep = selected(j);
                } else {
                    const int local = j - tb0;
                    const int ka = local / nbs, kb = local - ka * nbs;
                    const uint32_t cols = cover(kb);
                    for (uint32_t rows = cover(ka); rows != 0u && !keep; rows &= rows - 1u)
                        keep = (srows[wave][__builtin_ctz(rows)] & cols) != 0u;
                }
            }
            const uint64_t bal = __ballot(keep);
            if (keep) out[base + __popcll(bal & ((1ull << lane) - 1))] = j;
            base += __popcll(bal);
        }
    }
    for (int j = base + lane; j < nkbT; j += 64) out[j] = -1;
    if (lane == 0) a.kv_cnt[tg][(int64_t)bh * nqbT + qt] = base;
}

namespace {

size_t score_shmem(int parts, int stages, int head_dim, int nkb, int nq) {
    return (size_t)parts * stages * 32 * head_dim * 2 + parts * (size_t)(nkb / 2 + 2) * sizeof(ScoreChunk) +
           (size_t)(nkb + parts) * sizeof(int) + 12 + 2 * (size_t)nq * parts * sizeof(float) +
           (size_t)nkb * nq * sizeof(float);   // 12: padding to the 16-byte aligned float arrays
}

template <auto Kernel>
hipError_t launch_with_shmem(dim3 grid, dim3 block, size_t shmem, const ScoreArgs& a, hipStream_t stream) {
    const hipError_t e = allow_dynamic_lds<Kernel>(shmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(Kernel, grid, block, shmem, stream, a);
    return hipGetLastError();
}

constexpr size_t kLdsBytes = 160 * 1024;

}  // namespace

hipError_t launch_cs4a_score(const ScoreArgs& a, int head_dim, hipStream_t stream) {
    // two query tiles per workgroup with the deepest ring that fits one CU's LDS;
    // else (many key tiles) one tile per workgroup
    const dim3 grid2((unsigned)(((a.nqb + 1) / 2) * a.B * a.H)), block2(kScore2Threads);
    const size_t s4 = score_shmem(kScoreParts, 4, head_dim, a.nkb, 128);
    const size_t s3 = score_shmem(kScoreParts, 3, head_dim, a.nkb, 128);
    if (head_dim == 128) {
        if (s4 <= kLdsBytes) return launch_with_shmem<cs4a_score2_kernel<128, 4>>(grid2, block2, s4, a, stream);
        if (s3 <= kLdsBytes) return launch_with_shmem<cs4a_score2_kernel<128, 3>>(grid2, block2, s3, a, stream);
    } else {
        if (s4 <= kLdsBytes) return launch_with_shmem<cs4a_score2_kernel<64, 4>>(grid2, block2, s4, a, stream);
        if (s3 <= kLdsBytes) return launch_with_shmem<cs4a_score2_kernel<64, 3>>(grid2, block2, s3, a, stream);
    }
    const size_t shmem = score_shmem(kScoreParts, kScoreStages, head_dim, a.nkb, 64);
    const dim3 grid((unsigned)(a.nqb * a.B * a.H)), block(kScoreThreads);
    if (head_dim == 128) return launch_with_shmem<cs4a_score_kernel<128>>(grid, block, shmem, a, stream);
    return launch_with_shmem<cs4a_score_kernel<64>>(grid, block, shmem, a, stream);
}

hipError_t launch_cs4a_select_map(const SelMapArgs& a, int bh, hipStream_t stream) {
    hipLaunchKernelGGL(cs4a_select_map_kernel, dim3(bh * a.groups_total), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vs

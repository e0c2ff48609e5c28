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
// two wave pairs (even / odd tiles) whose maxima and sums are merged exactly
// at the end.  The QK^T work is the bf16 MFMA tile engine of the attention
// kernel.  Reductions run in a fixed order: scores are bit-reproducible.
//
// cs4a_select_map_kernel: one wave per (batch, head, target query tile).
// Top-p (or Top-K) on integer-quantised scores (exact, associative) of the
// parent decision tile, kept as a bitset in registers, then the target-scale lists: parent tile by floor scaling, tiles below the
// decision scale copied, decision-scale tiles expanded to their footprint on
// every scale from D to the target, sink tiles added.
#include "kernel_args.h"

namespace vs {

// Walk over the key tiles of one parity (tiles par, par + 2, ...), each in
// halves of up to 4 rows.
struct TileWalk {
    int j, half;
};

__device__ __forceinline__ bool tile_next(TileWalk& w, const DevGeom& g, int nkb, int& tile, int& base, int& stride,
                                          int& nrows, int& ncols) {
    if (w.j >= nkb) return false;
    const int s = scale_of_tile(g, w.j);
    const int local = w.j - g.tile_base[s];
    const int nb = g.nb[s], side = g.side[s];
    const int ta = local / nb, tb = local - ta * nb;
    const int rows = min(8, side - 8 * ta), cols = min(8, side - 8 * tb);
    tile = w.j;
    base = g.tok_off[s] + (8 * ta + 4 * w.half) * side + 8 * tb;
    stride = side;
    nrows = min(4, rows - 4 * w.half);
    ncols = cols;
    if (w.half == 0 && rows > 4) {
        w.half = 1;
    } else {
        w.half = 0;
        w.j += 2;
    }
    return true;
}

// Chunks of the tiles of one parity.
__device__ __forceinline__ int parity_chunks(const DevGeom& g, int nkb, int par) {
    int n = 0;
    for (int j = par; j < nkb; j += 2) {
        const int s = scale_of_tile(g, j);
        const int local = j - g.tile_base[s];
        const int ta = local / g.nb[s];
        n += (min(8, g.side[s] - 8 * ta) > 4) ? 2 : 1;
    }
    return n;
}

// Four waves per decision query tile: waves (2 par + qh) take query rows
// 4 qh .. 4 qh + 3 and the key tiles of parity par.  Each lane keeps, per key
// tile of its parity, the partial sum of exp2(s c - m) over its query's keys
// relative to its running max m (two lane halves of a query are summed into
// one LDS slot per chunk); at the end the two parities' maxima and sums are
// merged exactly, every partial is normalised by its query's total, and each
// key tile's score is summed over its 64 queries in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void cs4a_score_kernel(const ScoreArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int STAGE = 32 * ROWB;
    constexpr int RPL = 1024 / ROWB;
    constexpr int LOADS = 16 / RPL;
    constexpr float kLazy = 8.0f;
    extern __shared__ __attribute__((aligned(1024))) char dyn[];
    char* kst_base = dyn;                                  // [par][buf][STAGE]
    float* acc = (float*)(dyn + 4 * STAGE);                // [nkb][128]
    float* mrow = acc + a.nkb * 128;                       // [128]
    float* lrow = mrow + 128;                              // [128]

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qh = wave & 1, par = wave >> 1;
    const int n = lane & 31, g = lane >> 5;
    const int slot = (2 * par + qh) * 32 + n;              // one per (parity, query)
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

    for (int i = tid; i < nkb * 128; i += 256) acc[i] = 0.0f;
    const int nch0 = parity_chunks(a.g, nkb, 0), nch1 = parity_chunks(a.g, nkb, 1);
    const int nch = par ? nch1 : nch0, nmax = max(nch0, nch1);
    __syncthreads();
    wait_vmcnt(0);   // Q is in registers before LDS-DMA traffic starts

    const uint32_t kst0 = lds_addr(kst_base) + (uint32_t)(par * 2 * STAGE);
    auto load = [&](int base, int stride, int nrows, int ncols, uint32_t kst) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int row = 16 * qh + i * RPL + lane / CH;
            const int lc = (lane % CH) ^ swz<CH>(row);
            const int r = row >> 3, col = row & 7;
            const bool valid = r < nrows && col < ncols;
            const int t = valid ? base + r * stride + col : base;
            lds_dma16(kh + t * a.sk_t + lc * 8,
                      __builtin_amdgcn_readfirstlane(kst + (uint32_t)((16 * qh + i * RPL) * ROWB)));
        }
    };

    const float c = a.scale_log2;
    float m_run = -INFINITY;
    TileWalk walk{par, 0};
    int ct = 0, cb = 0, cs = 0, cr = 0, ccn = 0, nt = 0, nbs = 0, ns = 0, nr = 0, nc = 0;
    if (nch > 0) {
        tile_next(walk, a.g, nkb, ct, cb, cs, cr, ccn);
        load(cb, cs, cr, ccn, kst0);
    }
    // one workgroup barrier per step for all four waves; a parity with fewer
    // chunks runs empty steps
    for (int ci = 0; ci < nmax; ++ci) {
        wait_vmcnt(0);
        wg_barrier();
        const bool has = ci < nch;
        if (ci + 1 < nch) {
            tile_next(walk, a.g, nkb, nt, nbs, ns, nr, nc);
            load(nbs, ns, nr, nc, kst0 + (uint32_t)(((ci + 1) & 1) * STAGE));
        }
        if (has) {
            const char* kst = kst_base + par * 2 * STAGE + (ci & 1) * STAGE;
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
            float mx = sacc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float cand = mx * c;
            const bool need = cand > m_run + kLazy;
            if (__ballot(need)) {
                if (need) {
                    const float alpha = __builtin_amdgcn_exp2f(m_run - cand);
                    if (g == 0)
                        for (int kt = par; kt <= ct; kt += 2) acc[kt * 128 + slot] *= alpha;
                    m_run = cand;
                }
            }
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) part += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, -m_run));
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
            part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // both halves of the query's keys
            if (g == 0) acc[ct * 128 + slot] += part;
        }
        ct = nt; cb = nbs; cs = ns; cr = nr; ccn = nc;
    }

    // merge the two parities: common max M, total l, then normalise
    float l_mine = 0.0f;
    if (g == 0)
        for (int kt = par; kt < nkb; kt += 2) l_mine += acc[kt * 128 + slot];
    if (g == 0) {
        mrow[slot] = m_run;
        lrow[slot] = l_mine;
    }
    __syncthreads();
    if (g == 0) {
        const int other = (2 * (1 - par) + qh) * 32 + n;
        const float m_o = mrow[other];
        const float M = fmaxf(m_run, m_o);
        const float w_mine = __builtin_amdgcn_exp2f(m_run - M), w_o = __builtin_amdgcn_exp2f(m_o - M);
        const float l_q = l_mine * w_mine + lrow[other] * w_o;
        const float f = w_mine / l_q;
        for (int kt = par; kt < nkb; kt += 2) acc[kt * 128 + slot] *= f;
    }
    __syncthreads();
    float* out = a.scores + ((int64_t)bh * a.nqb + qt) * nkb;
    for (int kt = tid; kt < nkb; kt += 256) {
        const int p = kt & 1;
        float sum = 0.0f;
        for (int q = 0; q < 64; ++q) sum += acc[kt * 128 + (2 * p + (q >> 5)) * 32 + (q & 31)];
        out[kt] = sum * (1.0f / 64.0f);
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
// ballots.  The wave whose target tile is the first child of its parent also
// writes the parent's selection (sel_cnt / sel_idx) when asked to.
__global__ __launch_bounds__(256) void cs4a_select_map_kernel(const SelMapArgs a) {
    __shared__ int64_t mq[4][256];   // quantised scores of each wave's parent tile
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int groups = (a.nqbT + 3) / 4;
    const int bh = blockIdx.x / groups;
    const int qt = (blockIdx.x - bh * groups) * 4 + wave;
    if (qt >= a.nqbT) return;   // whole wave leaves; no workgroup barrier below
    const int nkbD = a.nkbD;
    const int D = a.d_scale, t = a.g.tile;
    const int hD = a.g.side[D], nbD = a.g.nb[D], nbT = a.g.nb[a.t_scale];
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
    if (a.sel_idx != nullptr && first_row && first_col) {
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

    // ---- mapping onto the target scale
    int base = 0;
    int32_t* out = a.kv_idx + ((int64_t)bh * a.nqbT + qt) * a.nkbT;
    for (int c0 = 0; c0 < a.nkbT; c0 += 64) {
        const int j = c0 + lane;
        bool keep = false;
        if (j < a.nkbT) {
            const int s = scale_of_tile(a.g, j);
            if (s < a.n_sink) {
                keep = true;
            } else if (s < D) {
                keep = selected(j);
            } else {
                const int hs = a.g.side[s], nbs = a.g.nb[s];
                const int local = j - a.g.tile_base[s];
                const int ka = local / nbs, kb = local - ka * nbs;
                const int klo_y = ka * t, khi_y = min(ka * t + t, hs) - 1;
                const int klo_x = kb * t, khi_x = min(kb * t + t, hs) - 1;
                for (int sa = 0; sa < nbD && !keep; ++sa) {
                    const int ey = min(sa * t + t, hD);
                    const int lo_y = (int)(((int64_t)sa * t * hs) / hD);
                    const int hi_y = (int)(((int64_t)ey * hs + hD - 1) / hD) - 1;
                    if (klo_y > hi_y || lo_y > khi_y) continue;
                    for (int sb = 0; sb < nbD; ++sb) {
                        if (!selected(a.g.tile_base[D] + sa * nbD + sb)) continue;
                        const int ex = min(sb * t + t, hD);
                        const int lo_x = (int)(((int64_t)sb * t * hs) / hD);
                        const int hi_x = (int)(((int64_t)ex * hs + hD - 1) / hD) - 1;
                        if (klo_x <= hi_x && lo_x <= khi_x) { keep = true; break; }
                    }
                }
            }
        }
        const uint64_t bal = __ballot(keep);
        if (keep) out[base + __popcll(bal & ((1ull << lane) - 1))] = j;
        base += __popcll(bal);
    }
    for (int j = base + lane; j < a.nkbT; j += 64) out[j] = -1;
    if (lane == 0) a.kv_cnt[(int64_t)bh * a.nqbT + qt] = base;
}

hipError_t launch_cs4a_score(const ScoreArgs& a, int head_dim, hipStream_t stream) {
    const int stage = 32 * head_dim * 2;
    const size_t shmem = 4 * (size_t)stage + (size_t)a.nkb * 128 * sizeof(float) + 256 * sizeof(float);
    dim3 grid((unsigned)(a.nqb * a.B * a.H)), block(256);
    if (head_dim == 128) {
        hipError_t e = hipFuncSetAttribute((const void*)cs4a_score_kernel<128>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cs4a_score_kernel<128>, grid, block, shmem, stream, a);
    } else {
        hipError_t e = hipFuncSetAttribute((const void*)cs4a_score_kernel<64>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cs4a_score_kernel<64>, grid, block, shmem, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_cs4a_select_map(const SelMapArgs& a, int bh, hipStream_t stream) {
    const int groups = (a.nqbT + 3) / 4;
    hipLaunchKernelGGL(cs4a_select_map_kernel, dim3(bh * groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vs

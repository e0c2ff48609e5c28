// CS4A: decision-scale block scores, top-p selection and cross-scale index
// mapping (SparVAR, ai.info summary, "Methodology in Plain English", first
// module; "Main Findings", the decision scale).
//
// cs4a_score_kernel: full attention of the decision scale's queries over the
// keys of scales 0..D, reduced to one number per (query tile, key tile): the
// mean over the tile's queries of the softmax mass falling in the key tile.
// Single pass: each lane keeps, per key tile, its partial sum of
// exp2(s*c - m) relative to its query's running max m (raised lazily, with
// the partial sums rescaled when it is), and the row total is the sum of the
// partials.  The QK^T work is the bf16 MFMA tile engine of the attention
// kernel.  Reductions run in a fixed order: scores are bit-reproducible.
//
// cs4a_select_map_kernel: one wave per (batch, head, target query tile).
// Top-p on integer-quantised scores (exact, associative) of the parent
// decision tile, kept as a bitset in registers, then the target-scale lists: parent tile by floor scaling, tiles below the
// decision scale copied, decision-scale tiles expanded to their footprint on
// every scale from D to the target, sink tiles added.
#include "kernel_args.h"

namespace vs {

template <int D>
__global__ __launch_bounds__(128) void cs4a_score_kernel(const ScoreArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr int STAGE = 32 * ROWB;
    constexpr int RPL = 1024 / ROWB;
    constexpr int LOADS = 16 / RPL;
    constexpr float kLazy = 8.0f;
    extern __shared__ __attribute__((aligned(1024))) char dyn[];
    char* kst_base = dyn;                              // [2][STAGE]
    float* acc = (float*)(dyn + 2 * STAGE);            // [nkb][128]

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, g = lane >> 5;
    const int bh = blockIdx.x / a.nqb, qt = blockIdx.x - bh * a.nqb;
    const int b = bh / a.H, h = bh - b * a.H;
    const int nkb = a.nkb;

    const int nbq = a.d_side >> 3;
    const int ti = qt / nbq, tj = qt - ti * nbq;
    const int64_t tok = (int64_t)(8 * ti + 4 * wave + (n >> 3)) * a.d_side + 8 * tj + (n & 7);
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;

    for (int i = tid; i < nkb * 128; i += 128) acc[i] = 0.0f;
    __syncthreads();
    wait_vmcnt(0);   // Q is in registers before LDS-DMA traffic starts

    // walk every key tile, in halves of up to 4 rows
    int j = 0, half = 0;
    auto next = [&](int& tile_id, int& base, int& stride, int& nrows, int& ncols) -> bool {
        if (j >= nkb) return false;
        const int s = scale_of_tile(a.g, j);
        const int local = j - a.g.tile_base[s];
        const int nb = a.g.nb[s], side = a.g.side[s];
        const int ta = local / nb, tb = local - ta * nb;
        const int rows = min(8, side - 8 * ta), cols = min(8, side - 8 * tb);
        tile_id = j;
        base = a.g.tok_off[s] + (8 * ta + 4 * half) * side + 8 * tb;
        stride = side;
        nrows = min(4, rows - 4 * half);
        ncols = cols;
        if (half == 0 && rows > 4) half = 1;
        else { half = 0; ++j; }
        return true;
    };
    auto load = [&](int base, int stride, int nrows, int ncols, uint32_t kst) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int row = 16 * wave + i * RPL + lane / CH;
            const int lc = (lane % CH) ^ swz<CH>(row);
            const int r = row >> 3, col = row & 7;
            const bool valid = r < nrows && col < ncols;
            const int t = valid ? base + r * stride + col : base;
            lds_dma16(kh + t * a.sk_t + lc * 8,
                      __builtin_amdgcn_readfirstlane(kst + (uint32_t)((16 * wave + i * RPL) * ROWB)));
        }
    };

    const float c = a.scale_log2;
    float m_run = -INFINITY;
    const int slot = tid;
    int ct, cb, cs, cr, ccn, nt, nbs, ns, nr, nc;
    bool have = next(ct, cb, cs, cr, ccn);
    const uint32_t kst0 = lds_addr(kst_base);
    if (have) load(cb, cs, cr, ccn, kst0);
    int buf = 0;
    while (have) {
        const bool more = next(nt, nbs, ns, nr, nc);
        if (more) load(nbs, ns, nr, nc, kst0 + (buf ^ 1) * STAGE);
        wait_vmcnt(more ? LOADS : 0);
        wg_barrier();
        const char* kst = kst_base + buf * STAGE;
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
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float cand = mx * c;
        const bool need = cand > m_run + kLazy;
        if (__ballot(need)) {
            if (need) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - cand);
                for (int kt = 0; kt <= ct; ++kt) acc[kt * 128 + slot] *= alpha;
                m_run = cand;
            }
        }
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, -m_run));
        acc[ct * 128 + slot] += part;
        wg_barrier();
        ct = nt; cb = nbs; cs = ns; cr = nr; ccn = nc;
        have = more;
        buf ^= 1;
    }

    // normalise each lane's partials by its query's total, then sum per key tile
    float l_lane = 0.0f;
    for (int kt = 0; kt < nkb; ++kt) l_lane += acc[kt * 128 + slot];
    const float l_q = l_lane + __shfl_xor(l_lane, 32);
    const float inv = 1.0f / l_q;
    for (int kt = 0; kt < nkb; ++kt) acc[kt * 128 + slot] *= inv;
    __syncthreads();
    float* out = a.scores + ((int64_t)bh * a.nqb + qt) * nkb;
    for (int kt = tid; kt < nkb; kt += 128) {
        float sum = 0.0f;
        for (int s = 0; s < 128; ++s) sum += acc[kt * 128 + s];
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
                int64_t before = 0;
                for (int i = 0; i < nkbD; ++i) {
                    const int64_t mi = mq[wave][i];
                    before += (mi > mj || (mi == mj && i < j)) ? mi : 0;
                }
                keep = (double)before < thr;
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
    const size_t shmem = 2 * (size_t)stage + (size_t)a.nkb * 128 * sizeof(float);
    dim3 grid((unsigned)(a.nqb * a.B * a.H)), block(128);
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

// Block-sparse (and dense) flash-style attention forward, bf16 in / bf16 out,
// fp32 accumulation, for gfx950 (CDNA4).
//
// What it computes: SparVAR's block-wise sparse attention (ai.info summary,
// "Key Contributions" item 3, "Main Findings" last item): each query tile of
// the query scale attends only to the tokens of its kept key tiles, with an
// ordinary scaled-dot-product softmax.  The dense variant walks every key.
//
// Design (MI355X-first, not the pages' FlexAttention kernel):
//  * one workgroup = one 8x8 query tile (64 queries) of one (batch, head);
//    two waves, each owning 4 query rows (32 queries);
//  * keys are consumed in chunks of 32: half a key tile (4 rows of <= 8
//    tokens), or 32 consecutive tokens of the leading run of wholly kept
//    scales (the sink scales are contiguous in the cache, so their small tiles
//    are packed instead of padded);
//  * the kept-tile list is decoded 64 entries at a time, one entry per lane
//    (token base, row stride, rows, cols), and read back per chunk with
//    readlane, so the walk itself costs a few scalar instructions per chunk;
//  * K and V chunks go HBM -> LDS with gfx950's 16-byte-per-lane direct loads
//    (global_load_lds_dwordx4, 64-bit head base in SGPRs, 32-bit lane offset:
//    one VALU add per load), double buffered, rows XOR-swizzled in 16-byte
//    units so that the MFMA operand reads below are bank-conflict free;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in
//    registers for the whole walk), so that every lane holds the scores of a
//    single query: the row max needs one v_permlane32_swap, row sums none;
//  * online softmax in the exp2 domain; the running max is only raised when a
//    new score exceeds it by more than 2^8 in the exponent (exact in
//    arithmetic: the final normalisation uses the same stale max);
//  * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator registers (no data movement), V^T is read from LDS with
//    gfx950's transposing ds_read_b64_tr_b16.
#include "kernel_args.h"

namespace vs {

// One chunk of up to 32 keys: key slot k (0..31) is token
// base + (k/8)*stride + (k%8), valid iff k/8 < nrows, k%8 < ncols, k < nvalid.
struct Chunk {
    int32_t base, stride, nrows, ncols, nvalid;
};

// Walk state over the kept keys of one query tile.  Lane i of desc0/desc1
// holds the decoded list entry cache_base + i: token base of the tile, and
// stride | rows << 16 | cols << 24.
struct Cursor {
    int32_t cnext, cend;   // leading contiguous token run [cnext, cend)
    int32_t j, cnt;        // position in the kept-tile list
    int32_t half;          // which half (rows 0-3 / 4-7) of tile j comes next
    const int32_t* idx;
    int32_t cache_base;
    int32_t desc0, desc1;
};

// Decode list entries cache_base .. cache_base+63 (one per lane).  Entries are
// documented to be valid tile ids; out-of-range ids are clamped so that a bad
// list cannot address outside the cache.
__device__ __forceinline__ void cursor_fill(Cursor& c, const DevGeom& g, int lane) {
    c.cache_base = c.j;
    const int e = c.j + lane;
    int id = e < c.cnt ? c.idx[e] : 0;
    id = min(max(id, 0), g.tile_base[g.n_scales] - 1);
    int tb = 0, side = g.side[0], off = 0, nb = g.nb[0];
    for (int s = 1; s < g.n_scales; ++s) {
        if (id >= g.tile_base[s]) {
            tb = g.tile_base[s];
            side = g.side[s];
            off = g.tok_off[s];
            nb = g.nb[s];
        }
    }
    const int local = id - tb;
    int a = (int)(((float)local + 0.5f) / (float)nb);
    a -= (a * nb > local);
    a += ((a + 1) * nb <= local);
    const int b = local - a * nb, t = g.tile;
    const int rows = min(t, side - a * t), cols = min(t, side - b * t);
    c.desc0 = off + a * t * side + b * t;
    c.desc1 = side | (rows << 16) | (cols << 24);
}

__device__ __forceinline__ bool cursor_next(Cursor& c, const DevGeom& g, Chunk& out, int lane) {
    if (c.cnext < c.cend) {
        out.base = c.cnext;
        out.stride = 8;
        out.nrows = 4;
        out.ncols = 8;
        out.nvalid = min(32, c.cend - c.cnext);
        c.cnext += 32;
        return true;
    }
    if (c.j >= c.cnt) return false;
    if (c.j - c.cache_base >= 64) cursor_fill(c, g, lane);
    const int slot = c.j - c.cache_base;
    const int base = __builtin_amdgcn_readlane(c.desc0, slot);
    const int info = __builtin_amdgcn_readlane(c.desc1, slot);
    const int side = info & 0xffff, rows = (info >> 16) & 0xff, cols = info >> 24;
    const int r0 = 4 * c.half;
    out.base = base + r0 * side;
    out.stride = side;
    out.nrows = min(4, rows - r0);
    out.ncols = cols;
    out.nvalid = 32;
    if (c.half == 0 && rows > 4) {
        c.half = 1;
    } else {
        c.half = 0;
        ++c.j;
    }
    return true;
}

// Per-lane constants of the chunk loads.  A wave fills key rows
// [16 wave, 16 wave + 16) of a stage; load i covers RPL consecutive rows, whose
// chunk row (key slot / 8) is the same for the whole wave.
template <int D>
struct LoadPlan {
    static constexpr int ROWB = D * 2;          // LDS bytes per key row
    static constexpr int CH = D / 8;            // 16-byte units per row
    static constexpr int RPL = 1024 / ROWB;     // rows per wave-wide load
    static constexpr int LOADS = 16 / RPL;      // loads per wave per tensor
    int32_t kc[LOADS], vc[LOADS];   // col * row_bytes + unit offset (K, V)
    int32_t lu[LOADS];              // unit offset alone (clamped slots)
    int32_t col[LOADS];             // token column within the chunk row
    int32_t slot[LOADS];            // key slot 0..31
};

template <int D>
__device__ __forceinline__ void make_plan(LoadPlan<D>& p, int wave, int lane, int64_t sk_t, int64_t sv_t) {
    using P = LoadPlan<D>;
#pragma unroll
    for (int i = 0; i < P::LOADS; ++i) {
        const int row = 16 * wave + i * P::RPL + lane / P::CH;
        const int unit = (lane % P::CH) ^ swz<P::CH>(row);
        p.slot[i] = row;
        p.col[i] = row & 7;
        p.lu[i] = unit * 16;
        p.kc[i] = (row & 7) * (int32_t)(sk_t * 2) + unit * 16;
        p.vc[i] = (row & 7) * (int32_t)(sv_t * 2) + unit * 16;
        // opaque to the optimizer: keeps the per-chunk address at one add
        // instead of a re-associated per-lane multiply
        asm volatile("" : "+v"(p.kc[i]), "+v"(p.vc[i]), "+v"(p.lu[i]));
    }
}

template <int D>
__device__ __forceinline__ void load_chunk(const LoadPlan<D>& p, const __bf16* kh, const __bf16* vh, int32_t krb,
                                           int32_t vrb, const Chunk& c, uint32_t k_lds, uint32_t v_lds,
                                           int wave) {
    using P = LoadPlan<D>;
    const bool full = c.nrows == 4 && c.ncols == 8 && c.nvalid == 32;
#pragma unroll
    for (int i = 0; i < P::LOADS; ++i) {
        const int r = (16 * wave + i * P::RPL) >> 3;     // chunk row of this load (wave-uniform)
        const int32_t ks = (c.base + r * c.stride) * krb, vs_ = (c.base + r * c.stride) * vrb;
        int32_t ko = ks + p.kc[i], vo = vs_ + p.vc[i];
        if (!full) {
            const bool valid = r < c.nrows && p.col[i] < c.ncols && p.slot[i] < c.nvalid;
            ko = valid ? ko : c.base * krb + p.lu[i];
            vo = valid ? vo : c.base * vrb + p.lu[i];
        }
        const uint32_t dst = (uint32_t)((16 * wave + i * P::RPL) * P::ROWB);
        lds_dma16_off(kh, ko, __builtin_amdgcn_readfirstlane(k_lds + dst));
        lds_dma16_off(vh, vo, __builtin_amdgcn_readfirstlane(v_lds + dst));
    }
}

// Everything one wave carries across chunks.
template <int D>
struct WaveState {
    bf16x8 qreg[D / 16];          // B operand of S^T = K Q^T (this lane's query)
    f32x16 oacc[D / 32];          // O^T accumulator
    float m_run, l_run;           // running max (log2 domain) and this lane's partial sum
};

// max / sum of a value and its partner lane (lane ^ 32) via v_permlane32_swap
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Consume one chunk of 32 keys from LDS (kst: K rows, vst: V rows).
template <int D>
__device__ __forceinline__ void attend_chunk(WaveState<D>& st, const char* __restrict__ kst,
                                             const char* __restrict__ vst, const Chunk& cc, float c, int lane) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    constexpr float kLazy = 8.0f;
    const int n = lane & 31, g = lane >> 5;

    // S^T (32 keys x 32 queries) = K Q^T
    f32x16 sacc = (f32x16)0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const int pc = (2 * s + g) ^ swz<CH>(n);
        const bf16x8 kop = *(const bf16x8*)(kst + n * ROWB + pc * 16);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, st.qreg[s], sacc, 0, 0, 0);
    }
    // padding keys of partial chunks -> -inf (value i sits at row i/4, column 4g + i%4)
    if (cc.nrows < 4 || cc.ncols < 8 || cc.nvalid < 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i >> 2, col = 4 * g + (i & 3), key = 8 * r + col;
            if (!(r < cc.nrows && col < cc.ncols && key < cc.nvalid)) sacc[i] = -INFINITY;
        }
    }
    // online softmax (log2 domain), running max raised lazily
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    mx = half_swap_max(mx);
    const float cand = mx * c;
    const bool need = cand > st.m_run + kLazy;
    if (__ballot(need)) {
        const float m_new = need ? cand : st.m_run;
        const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= alpha;
        st.l_run *= alpha;
        st.m_run = m_new;
    }
    bf16x8 pt[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, -st.m_run));
        st.l_run += p;
        pt[i >> 3][i & 7] = (__bf16)p;
    }
    // O^T (D x 32 queries) += V^T P^T, V^T through transposing LDS reads
    const int c16 = lane >> 4, p16 = lane & 15;
    const int half = c16 & 1, r4 = p16 >> 2, q4 = p16 & 3;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
        const int d = 32 * mb + 16 * half + 4 * q4;
        const int lc = d >> 3, within = (d & 7) * 2;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x4 part[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int row = 16 * t + 8 * jj + 4 * g + r4;
                const char* addr = vst + row * ROWB + ((lc ^ swz<CH>(row)) << 4) + within;
                part[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(addr));
            }
            const bf16x8 vop = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
            st.oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pt[t], st.oacc[mb], 0, 0, 0);
        }
    }
}

template <int D, bool DENSE>
__global__ __launch_bounds__(128, 2) void attn_fwd_bf16_kernel(const AttnArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int STAGE = 32 * D * 2;
    constexpr int LOADS = 2 * LoadPlan<D>::LOADS;   // vm instructions per wave per chunk
    __shared__ __attribute__((aligned(1024))) char smem[4 * STAGE];   // [stage][K, V]

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 31, g = lane >> 5;  // query column and lane half of this lane

    const int64_t nqt = DENSE ? (a.nq + 63) / 64 : a.nqb;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = work / nqt, qt = work - bh * nqt;
    const int b = bh / a.H, h = bh - b * a.H;

    // ---- the query this lane holds (column n of the wave's 32 queries)
    int64_t tok;
    bool qvalid = true;
    if (DENSE) {
        tok = 64 * (int64_t)qt + 32 * wave + n;
        qvalid = tok < a.nq;
        if (!qvalid) tok = a.nq - 1;
    } else {
        const int nbq = a.q_side >> 3;
        const int ti = qt / nbq, tj = qt - ti * nbq;
        tok = (int64_t)(8 * ti + 4 * wave + (n >> 3)) * a.q_side + 8 * tj + (n & 7);
    }
    WaveState<D> st;
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) st.qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] = (f32x16)0.0f;
    st.m_run = -INFINITY;
    st.l_run = 0.0f;
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;
    const __bf16* vh = a.v + b * a.sv_b + h * a.sv_h;
    const int32_t krb = (int32_t)(a.sk_t * 2), vrb = (int32_t)(a.sv_t * 2);
    LoadPlan<D> plan;
    make_plan<D>(plan, wave, lane, a.sk_t, a.sv_t);

    // ---- kept-key walk
    Cursor cur;
    cur.half = 0;
    if (DENSE) {
        cur.cnext = 0;
        cur.cend = (int32_t)a.nk;
        cur.j = cur.cnt = 0;
        cur.idx = nullptr;
        cur.cache_base = 0;
        cur.desc0 = cur.desc1 = 0;
    } else {
        const int64_t row = (a.per_head ? (int64_t)bh * a.nqb : 0) + qt;
        cur.cnt = a.kv_cnt[row];
        cur.idx = a.kv_idx + row * a.nkb;
        // leading run of tiles 0,1,2,...: whole scales kept from the start form
        // one contiguous token range
        int p = 0;
        for (;;) {
            const int v = (p + lane < cur.cnt) ? cur.idx[p + lane] : -1;
            const uint64_t off = __ballot(v != p + lane);
            if (off) {
                p += __builtin_ctzll(off);
                break;
            }
            p += 64;
        }
        int s = 0;
        while (s < a.g.n_scales && a.g.tile_base[s + 1] <= p) ++s;
        cur.cnext = 0;
        cur.cend = a.g.tok_off[s];
        cur.j = a.g.tile_base[s];
        cursor_fill(cur, a.g, lane);
    }
    wait_vmcnt(0);   // Q and the first list entries are in registers before LDS-DMA traffic starts
    const float c = a.scale_log2;

    const uint32_t lds0 = lds_addr(smem);
    const char* sm = smem;
    Chunk cc, cn;
    bool have = cursor_next(cur, a.g, cc, lane);
    if (have) load_chunk<D>(plan, kh, vh, krb, vrb, cc, lds0, lds0 + STAGE, wave);
    while (have) {
        // stage 0 holds chunk cc; prefetch the next one into stage 1
        bool more = cursor_next(cur, a.g, cn, lane);
        if (more) {
            load_chunk<D>(plan, kh, vh, krb, vrb, cn, lds0 + 2 * STAGE, lds0 + 3 * STAGE, wave);
            wait_vmcnt(LOADS);
        } else {
            wait_vmcnt(0);
        }
        wg_barrier();
        attend_chunk<D>(st, sm, sm + STAGE, cc, c, lane);
        wg_barrier();
        if (!more) break;
        cc = cn;
        // stage 1 holds chunk cc; prefetch the next one into stage 0
        more = cursor_next(cur, a.g, cn, lane);
        if (more) {
            load_chunk<D>(plan, kh, vh, krb, vrb, cn, lds0, lds0 + STAGE, wave);
            wait_vmcnt(LOADS);
        } else {
            wait_vmcnt(0);
        }
        wg_barrier();
        attend_chunk<D>(st, sm + 2 * STAGE, sm + 3 * STAGE, cc, c, lane);
        wg_barrier();
        cc = cn;
        have = more;
    }

    // ---- epilogue
    const float l_tot = half_swap_sum(st.l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qvalid) {
        __bf16* op = a.o + b * a.so_b + h * a.so_h + tok * a.so_t;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (__bf16)(st.oacc[mb][4 * kk + e] * inv);
                *(bf16x4*)(op + 32 * mb + 8 * kk + 4 * g) = val;
            }
        }
        if (a.lse != nullptr && g == 0) {
            const int64_t nq_tot = DENSE ? a.nq : (int64_t)a.q_side * a.q_side;
            a.lse[(int64_t)bh * nq_tot + tok] =
                l_tot > 0.0f ? (st.m_run + __builtin_log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
    }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool dense, hipStream_t stream) {
    const int64_t nqt = dense ? (a.nq + 63) / 64 : a.nqb;
    const int64_t blocks = nqt * a.B * a.H;
    dim3 grid((unsigned)blocks), block(128);
    if (head_dim == 128) {
        if (dense) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), grid, block, 0, stream, a);
    } else {
        if (dense) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vs

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
//  * online softmax in the exp2 domain against a running maximum set by the
//    walk's first chunk: later chunks' weights go to the PV product with no
//    maximum over the chunk; a query whose weights in a chunk sum above 2^16
//    then has its maximum raised by ceil(log2 sum) and O and the row sum
//    scaled by that exact power of two; a weight that overflows leaves a
//    non-finite value, found at the end of the walk, which is then redone in
//    an exact form that raises the maximum to each chunk's before its weights
//    (exact in arithmetic either way: the final normalisation uses the same
//    running maximum as the weights);
//  * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator registers (no data movement), V^T is read from LDS with
//    gfx950's transposing ds_read_b64_tr_b16;
//  * the 64-query walk is pipelined by one chunk: chunk c - 1's PV MFMAs are
//    interleaved with chunk c's softmax in one scheduling region, so that a
//    wave's own MFMA and VALU work overlap (see pipe_chunk).
#include "kernel_args.h"

namespace vs {

// One chunk of up to 32 keys: key slot k (0..31) is token
// base + (k/8)*stride + (k%8), valid iff k/8 < nrows, k%8 < ncols, k < nvalid.
// Packed as two words: base, and stride | nrows << 16 | ncols << 19 |
// nvalid << 23 | full << 29 (full: all 32 slots valid).
struct Chunk {
    int32_t base, stride, nrows, ncols, nvalid;
    bool full;
};

__device__ __forceinline__ uint32_t pack_info(int stride, int nrows, int ncols, int nvalid) {
    const uint32_t full = (nrows == 4 && ncols == 8 && nvalid == 32) ? 1u : 0u;
    return (uint32_t)stride | ((uint32_t)nrows << 16) | ((uint32_t)ncols << 19) | ((uint32_t)nvalid << 23) |
           (full << 29);
}

__device__ __forceinline__ Chunk unpack_chunk(int32_t base, uint32_t info) {
    Chunk c;
    c.base = base;
    c.stride = info & 0xffff;
    c.nrows = (info >> 16) & 7;
    c.ncols = (info >> 19) & 15;
    c.nvalid = (info >> 23) & 63;
    c.full = (info >> 29) & 1;
    return c;
}

constexpr int kTableCap = 512;   // chunk descriptors per table build

// Walk state of one query tile: what remains to be put into the table.
struct Walk {
    int32_t cnext, cend;   // leading contiguous token run [cnext, cend)
    int32_t j, cnt;        // next list entry, list length
    const int32_t* idx;
};

// The geometry of scale `lane` held by that lane (lanes past the last scale:
// tile_base / tok_off = the totals, then INT_MAX), read once per workgroup:
// the decoding below takes each scale's figures with readlane instead of a
// chain of dependent scalar loads from the kernel arguments.
struct LaneGeom {
    int32_t tb, off, side, nb;
};

__device__ __forceinline__ LaneGeom lane_geom(const DevGeom& g, int lane) {
    LaneGeom lg;
    const int s = min(lane, kMaxScales - 1);
    lg.tb = lane <= g.n_scales ? g.tile_base[min(lane, kMaxScales)] : INT_MAX;
    lg.off = lane <= g.n_scales ? g.tok_off[min(lane, kMaxScales)] : INT_MAX;
    lg.side = lane < g.n_scales ? g.side[s] : 0;
    lg.nb = lane < g.n_scales ? g.nb[s] : 1;
    return lg;
}

// Wave 0 fills the chunk table with the next descriptors of the walk (the
// contiguous run first, then tile halves in list order) and returns how many
// it wrote; list entries are decoded one per lane and placed with a
// ballot prefix sum (every entry gives 1 or 2 chunks).  Entries are
// documented to be valid tile ids; out-of-range ids are clamped so that a bad
// list cannot address outside the cache.  `first64` holds list entries
// 0..63 (entry `lane` in lane `lane`, where the list has it) when
// `have_first64`: entries among them are taken from registers, not memory.
__device__ __forceinline__ int build_table(Walk& w, const DevGeom& g, const LaneGeom& lg, uint2* table, int lane,
                                           int first64 = 0, bool have_first64 = false) {
    int n = 0;
    if (w.cnext < w.cend) {
        const int nc = min((w.cend - w.cnext + 31) >> 5, kTableCap);
        for (int k = lane; k < nc; k += 64) {
            const int base = w.cnext + 32 * k;
            table[k] = make_uint2((uint32_t)base, pack_info(8, 4, 8, min(32, w.cend - base)));
        }
        w.cnext = min(w.cend, w.cnext + 32 * nc);
        n = nc;
    }
    const int n_tiles = __builtin_amdgcn_readlane(lg.tb, g.n_scales);
    while (w.j < w.cnt && kTableCap - n >= 128) {
        const int e = w.j + lane;
        const bool valid = e < w.cnt;
        const int from_regs = __builtin_amdgcn_ds_bpermute((e & 63) << 2, first64);
        int id = e;   // no list: every tile
        if (have_first64 && e < 64) id = from_regs;
        else if (valid && w.idx != nullptr) {
            id = w.idx[e];
            // consumed here: the wait for this load stays on this path (an
            // unconditional wait after the branch would also wait for the
            // first chunk's LDS-DMA loads issued before the table build)
            asm volatile("" : "+v"(id));
        }
        if (!valid) id = 0;
        id = min(max(id, 0), n_tiles - 1);
        int tb = 0, side = __builtin_amdgcn_readlane(lg.side, 0), off = 0, nb = __builtin_amdgcn_readlane(lg.nb, 0);
        for (int s = 1; s < g.n_scales; ++s) {
            const int tbs = __builtin_amdgcn_readlane(lg.tb, s);
            if (id >= tbs) {
                tb = tbs;
                side = __builtin_amdgcn_readlane(lg.side, s);
                off = __builtin_amdgcn_readlane(lg.off, s);
                nb = __builtin_amdgcn_readlane(lg.nb, s);
            }
        }
        const int local = id - tb;
        int a = (int)(((float)local + 0.5f) / (float)nb);
        a -= (a * nb > local);
        a += ((a + 1) * nb <= local);
        const int b = local - a * nb, t = g.tile;
        const int rows = min(t, side - a * t), cols = min(t, side - b * t);
        const int base = off + a * t * side + b * t;
        const bool two = valid && rows > 4;
        const uint64_t vb = __ballot(valid), tb2 = __ballot(two);
        const uint64_t lt = (1ull << lane) - 1;
        const int pos = n + __popcll(vb & lt) + __popcll(tb2 & lt);
        if (valid) {
            table[pos] = make_uint2((uint32_t)base, pack_info(side, min(4, rows), cols, 32));
            if (two) table[pos + 1] = make_uint2((uint32_t)(base + 4 * side), pack_info(side, rows - 4, cols, 32));
        }
        n += __popcll(vb) + __popcll(tb2);
        w.j = min(w.cnt, w.j + 64);
    }
    return n;
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
};

template <int D>
__device__ __forceinline__ int plan_slot(int wave, int lane, int i) {
    using P = LoadPlan<D>;
    return 16 * wave + i * P::RPL + lane / P::CH;          // key slot 0..31 filled by this lane
}

template <int D>
__device__ __forceinline__ int plan_unit(int slot, int lane) {
    using P = LoadPlan<D>;
    return (lane % P::CH) ^ swz<P::CH>(slot);             // swizzled 16-byte unit
}

template <int D>
__device__ __forceinline__ void make_plan(LoadPlan<D>& p, int wave, int lane, int64_t sk_t, int64_t sv_t) {
    using P = LoadPlan<D>;
#pragma unroll
    for (int i = 0; i < P::LOADS; ++i) {
        const int row = plan_slot<D>(wave, lane, i);
        const int unit = plan_unit<D>(row, lane);
        p.kc[i] = (row & 7) * (int32_t)(sk_t * 2) + unit * 16;
        p.vc[i] = (row & 7) * (int32_t)(sv_t * 2) + unit * 16;
        // opaque to the optimizer: keeps the per-chunk address at one add
        // instead of a re-associated per-lane multiply
        asm volatile("" : "+v"(p.kc[i]), "+v"(p.vc[i]));
    }
}

template <int D>
__device__ __forceinline__ void load_chunk(const LoadPlan<D>& p, const __bf16* kh, const __bf16* vh, int32_t krb,
                                           int32_t vrb, const Chunk& c, lds_ptr k_lds, lds_ptr v_lds,
                                           int wave, int lane) {
    using P = LoadPlan<D>;
    if (c.full) {
#pragma unroll
        for (int i = 0; i < P::LOADS; ++i) {
            const int r = (16 * wave + i * P::RPL) >> 3;     // chunk row of this load (wave-uniform)
            const int32_t t0 = c.base + r * c.stride;
            const int dst = (16 * wave + i * P::RPL) * P::ROWB;
            dma16(kh, (uint32_t)(t0 * krb + p.kc[i]), k_lds + dst);
            dma16(vh, (uint32_t)(t0 * vrb + p.vc[i]), v_lds + dst);
        }
    } else {
#pragma unroll
        for (int i = 0; i < P::LOADS; ++i) {
            const int slot = plan_slot<D>(wave, lane, i);
            const int r = slot >> 3, col = slot & 7;
            const int unit16 = plan_unit<D>(slot, lane) * 16;
            // padding slots re-read the chunk's first token (finite values; masked later)
            const bool valid = r < c.nrows && col < c.ncols && slot < c.nvalid;
            const int32_t tok = valid ? c.base + r * c.stride + col : c.base;
            const int dst = (16 * wave + i * P::RPL) * P::ROWB;
            dma16(kh, (uint32_t)(tok * krb + unit16), k_lds + dst);
            dma16(vh, (uint32_t)(tok * vrb + unit16), v_lds + dst);
        }
    }
}

// Everything one wave carries across chunks.
template <int D>
struct WaveState {
    bf16x8 qreg[D / 16];          // B operand of S^T = K Q^T (this lane's query)
    f32x16 oacc[D / 32];          // O^T accumulator
    float m_run, l_run;           // running max (log2 domain) and this lane's partial sum
    // this lane's byte offsets, within a stage, of its MFMA operand reads:
    // K rows (one per k-step) and V^T (transposing reads); a stage's own
    // offset is a compile-time constant added to them, which the LDS reads
    // take as their immediate offset
    uint32_t koff[D / 16];
    uint32_t voff[D / 32][2];     // rows 16 t + ..: the swizzle repeats every 16 rows, so t adds 16 rows

    // Called where the wave is about to wait for all its loads anyway: an
    // empty asm that reads and rewrites the Q^T operands tells the compiler
    // that their loads are complete.  Otherwise its own wait for them stays
    // in front of the S^T MFMAs of every chunk step, and a vmcnt wait there
    // also waits for the chunk loads issued after the barrier (asm, which the
    // compiler does not count).
    __device__ __forceinline__ void q_ready() {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(qreg[s]));
    }
};

// Fill the operand-read offsets of WaveState (once per kernel).  The values
// are made opaque to the compiler so that it keeps one register per read
// and adds each stage's constant in the instruction, instead of splitting
// them into a row part and a unit part that it re-adds for every chunk.
template <int D>
__device__ __forceinline__ void init_lds_offsets(WaveState<D>& st, int lane) {
    constexpr int ROWB = D * 2, CH = D / 8;
    const int n = lane & 31, g = lane >> 5;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        st.koff[s] = (uint32_t)(n * ROWB + (((2 * s + g) ^ swz<CH>(n)) << 4));
        asm volatile("" : "+v"(st.koff[s]));
    }
    const int c16 = lane >> 4, p16 = lane & 15;
    const int hf = c16 & 1, r4 = p16 >> 2, q4 = p16 & 3;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
        const int d = 32 * mb + 16 * hf + 4 * q4;
        const int lc = d >> 3, within = (d & 7) * 2;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int row = 8 * jj + 4 * g + r4;
            st.voff[mb][jj] = (uint32_t)(row * ROWB + ((lc ^ swz<CH>(row)) << 4) + within);
            asm volatile("" : "+v"(st.voff[mb][jj]));
        }
    }
}

// max / sum of a value and its partner lane (lane ^ 32) via v_permlane32_swap
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Weights of the fast softmax path stay at or below this (log2 domain: at most
// 16 above the running maximum), far inside the range of bf16 and float.
constexpr float kSumCap = 65536.0f;

template <bool V>
struct IntC {
    static constexpr bool value = V;
};

// P^T = exp2(S^T c - m) rounded to bf16 (the PV operand), and the lane's sum
// of the float weights (pairwise).
__device__ __forceinline__ float exp_chunk(const f32x16& s, float c, float m, bf16x8 (&pt)[2]) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
#pragma unroll
    for (int i = 0; i < 16; ++i) pt[i >> 3][i & 7] = (__bf16)p[i];
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = p[2 * i] + p[2 * i + 1];
    return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

// Consume one chunk of 32 keys from LDS (kst: K rows, vst: V rows).  The
// LDS operand reads of each phase are issued ahead of the MFMAs that consume
// them (all K rows before S^T, all V^T reads before the softmax, so they land
// while it runs); scheduling barriers keep the compiler from moving them back
// next to their uses.
template <int D, bool EXACT>
__device__ __forceinline__ void attend_chunk(WaveState<D>& st, const char* __restrict__ kst,
                                             const char* __restrict__ vst, const Chunk& cc, float c, int lane,
                                             uint32_t tokmask = 0xffffu) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int ROWB = D * 2;
    constexpr int CH = D / 8;
    const int n = lane & 31, g = lane >> 5;

    // S^T (32 keys x 32 queries) = K Q^T
    bf16x8 kop[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kop[s] = *(const bf16x8*)(kst + st.koff[s]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sacc = (f32x16)0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], st.qreg[s], sacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // V^T operands for the whole chunk (transposing LDS reads), in flight during the softmax
    bf16x8 vop[MBLK][2];
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x4 part[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const char* addr = vst + 16 * t * (2 * D) + st.voff[mb][jj];
                part[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(addr));
            }
            vop[mb][t] = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // keys outside the token-level mask (token-exact mode) -> -inf
    if (tokmask != 0xffffu) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (!((tokmask >> i) & 1u)) sacc[i] = -INFINITY;
    }
    // padding keys of partial chunks -> -inf (value i sits at row i/4, column 4g + i%4)
    if (!cc.full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i >> 2, col = 4 * g + (i & 3), key = 8 * r + col;
            if (!(r < cc.nrows && col < cc.ncols && key < cc.nvalid)) sacc[i] = -INFINITY;
        }
    }
    // online softmax (log2 domain).  EXACT (a walk's first chunk, and every
    // chunk of the safe pass): the running maximum is first raised to the
    // chunk's.  Otherwise the weights are taken
    // against the running maximum as it stands, with no maximum over the chunk:
    // weights up to 2^127 are finite in bf16 and float, so the product below
    // is exact in arithmetic; afterwards, when a query's weights in this chunk
    // sum above kSumCap, its maximum is raised by the integer ceil(log2 sum) and
    // O and the row sum scaled by the exact power of two, so later weights start
    // from at most 1 again.  A weight that overflows (a score more than 127
    // above the running maximum, log2 domain) leaves inf / NaN behind, which the
    // kernel detects at the end of the walk and answers with a safe pass.
    if (EXACT) {
        float mx = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        mx = half_swap_max(mx);
        const float m_new = fmaxf(st.m_run, mx * c);
        if (__builtin_amdgcn_ballot_w64(m_new > st.m_run)) {
            const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= alpha;
            st.l_run *= alpha;
            st.m_run = m_new;
        }
    }
    bf16x8 pt[2];
    const float sum = exp_chunk(sacc, c, st.m_run, pt);
    st.l_run += sum;
    __builtin_amdgcn_sched_barrier(0);

    // O^T (D x 32 queries) += V^T P^T
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
            st.oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[mb][t], pt[t], st.oacc[mb], 0, 0, 0);

    if (!EXACT && __builtin_amdgcn_ballot_w64(!(sum <= kSumCap))) {
        const float sq = half_swap_max(sum);               // both halves of the query agree
        if (sq > kSumCap && sq <= 3.0e38f) {
            const int dexp = (int)__builtin_ceilf(__builtin_log2f(sq));
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= __builtin_ldexpf(1.0f, -dexp);
            st.l_run = __builtin_ldexpf(st.l_run, -dexp);
            st.m_run += (float)dexp;
        }
    }
}

// ---- the pipelined chunk step of the 64-query walk
//
// One step takes chunk c's scores (K reads, S^T = K Q^T, masks) and then, in
// one scheduling region, chunk c - 1's product O^T += V^T P^T (its weights and
// V^T operands carried in registers from the previous step) interleaved with
// chunk c's weights, so that the wave's own MFMAs and softmax VALU overlap
// instead of running back to back.  Chunk c's V^T operands are read last, for
// its product in the next step.  A raise of the running maximum decided from
// chunk c's weights (the fast form) scales O^T after chunk c's product, i.e.
// in the next step or in the drain; the exact form scales O^T (after chunk
// c - 1's product) before chunk c's product.  A segment's first step takes a
// zero product (zero weights and zero V^T operands).
template <int D>
struct PipeState {
    bf16x8 pt[2];              // P^T of the chunk whose product is pending
    bf16x8 vop[D / 32][2];     // its V^T operands
    float pend;                // scale for O^T once that product is in (1: none)
};

template <int D, bool EXACT>
__device__ __forceinline__ void pipe_chunk(WaveState<D>& st, PipeState<D>& ps, const char* __restrict__ kst,
                                           const char* __restrict__ vst, const Chunk& cc, float c, int lane,
                                           uint32_t tokmask) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    const int g = lane >> 5;

    // S^T (32 keys x 32 queries) = K Q^T, the K operands read in two halves
    // (the second half's reads overlap the first half's MFMAs)
    constexpr int KH = KSTEPS / 2;
    f32x16 sacc = (f32x16)0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        bf16x8 kop[KH];
#pragma unroll
        for (int s = 0; s < KH; ++s) kop[s] = *(const bf16x8*)(kst + st.koff[KH * hh + s]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KH; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], st.qreg[KH * hh + s], sacc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    if (tokmask != 0xffffu) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (!((tokmask >> i) & 1u)) sacc[i] = -INFINITY;
    }
    if (!cc.full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = i >> 2, col = 4 * g + (i & 3), key = 8 * r + col;
            if (!(r < cc.nrows && col < cc.ncols && key < cc.nvalid)) sacc[i] = -INFINITY;
        }
    }
    float alpha = 1.0f;
    if (EXACT) {   // raise the running maximum to the chunk's first
        float mx = sacc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
        mx = half_swap_max(mx);
        const float m_new = fmaxf(st.m_run, mx * c);
        alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
        st.m_run = m_new;
    }

    // chunk c - 1's product interleaved with chunk c's weights
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c, -st.m_run));
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
            st.oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ps.vop[mb][t], ps.pt[t], st.oacc[mb], 0, 0, 0);
    bf16x8 pt[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pt[i >> 3][i & 7] = (__bf16)p[i];
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = p[2 * i] + p[2 * i + 1];
    float sum = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
    // the weights are computed here, beside the product, not sunk toward
    // their later uses
    asm volatile("" : "+v"(sum), "+v"(pt[0]), "+v"(pt[1]));
    // one MFMA, then a share of the weights' VALU work (16 fma, 16 exp, 8
    // packs, 15 adds), 2 MBLK times
#pragma unroll
    for (int k = 0; k < 2 * MBLK; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 56 / (2 * MBLK), 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // V^T operands of chunk c (transposing LDS reads), for its product in the next step
    // (chunk c - 1's product has read the registers they replace)
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x4 part[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
                part[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(vst + 16 * t * (2 * D) + st.voff[mb][jj]));
            ps.vop[mb][t] = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    if (EXACT) {
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= alpha;
        }
        st.l_run = st.l_run * alpha + sum;
    } else {
        if (__builtin_amdgcn_ballot_w64(ps.pend != 1.0f)) {
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= ps.pend;
        }
        st.l_run += sum;
        ps.pend = 1.0f;
        if (__builtin_amdgcn_ballot_w64(!(sum <= kSumCap))) {
            const float sq = half_swap_max(sum);               // both halves of the query agree
            if (sq > kSumCap && sq <= 3.0e38f) {
                const int dexp = (int)__builtin_ceilf(__builtin_log2f(sq));
                st.l_run = __builtin_ldexpf(st.l_run, -dexp);
                st.m_run += (float)dexp;
                ps.pend = __builtin_ldexpf(1.0f, -dexp);
            }
        }
    }

    ps.pt[0] = pt[0];
    ps.pt[1] = pt[1];
}

// No pending product: zero weights against zero V^T operands (a segment's
// first step then adds nothing to O^T).
template <int D>
__device__ __forceinline__ void pipe_reset(PipeState<D>& ps) {
    const bf16x8 z = (bf16x8)(__bf16)0.0f;
    ps.pt[0] = ps.pt[1] = z;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) ps.vop[mb][0] = ps.vop[mb][1] = z;
    ps.pend = 1.0f;
}

// The pending product and O^T scale at the end of a walk segment.
template <int D>
__device__ __forceinline__ void pipe_drain(WaveState<D>& st, PipeState<D>& ps) {
    constexpr int MBLK = D / 32;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
            st.oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ps.vop[mb][t], ps.pt[t], st.oacc[mb], 0, 0, 0);
    if (__builtin_amdgcn_ballot_w64(ps.pend != 1.0f)) {
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= ps.pend;
    }
    pipe_reset<D>(ps);
}

// floor(num / den) for 0 <= num < 2^24, den >= 1 (float estimate, one correction each way)
__device__ __forceinline__ int div_floor(int num, int den) {
    int q = (int)((float)num / (float)den);
    q -= (q * den > num);
    q += ((q + 1) * den <= num);
    return q;
}

// Token mode: per-wave constants of the CSLA rule and the projection of this
// lane's query onto the scale of the chunks being walked.  Lane s holds the
// side, token offset and radius of scale s; chunks arrive in ascending
// order, so the projection is recomputed only when the scale changes (the
// chunk's row stride is its scale's side, and sides are strictly
// ascending, so the stride names the scale).
struct TokenState {
    int32_t sink_end;              // first token after the sink scales
    int32_t lside, ltok, lrad;     // this lane's scale (lanes >= n_scales: side 0)
    int32_t side, off, r, py, px;  // the current chunk scale (side 0: none yet)
};

__device__ __forceinline__ void token_init(TokenState& ts, const AttnArgs& a, int lane) {
    ts.lside = ts.ltok = ts.lrad = 0;
    for (int s = 0; s < a.g.n_scales; ++s) {
        if (lane == s) {
            ts.lside = a.g.side[s];
            ts.ltok = a.g.tok_off[s];
            ts.lrad = a.radius[s];
        }
    }
    ts.sink_end = __builtin_amdgcn_readlane(ts.ltok, a.n_sink < a.g.n_scales ? a.n_sink : 0);
    if (a.n_sink >= a.g.n_scales) ts.sink_end = a.g.tok_off[a.g.n_scales];
    ts.side = 0;
    ts.off = ts.r = ts.py = ts.px = 0;
}

// Token-level CSLA keep bits of a tile-half chunk for this lane (value i at
// key row i/4, column 4g + i%4 of the chunk): a key of scale s at (y', x') is
// kept iff s is a sink scale, or radius[s] >= 0 and |y' - floor(qy h_s / H)|
// and |x' - floor(qx h_s / H)| are both <= radius[s] (SparVAR, ai.info
// summary, "Methodology in Plain English", second module).  Chunks of sink
// scales keep every key.
__device__ __forceinline__ uint32_t csla_token_bits(TokenState& ts, const Chunk& c, int qy, int qx, int q_side,
                                                    int g) {
    if (c.base < ts.sink_end) return 0xffffu;
    if (c.stride != ts.side) {
        const uint64_t m = __ballot(ts.lside == c.stride);
        const int s = m ? __builtin_ctzll(m) : 0;
        ts.side = c.stride;
        ts.off = __builtin_amdgcn_readlane(ts.ltok, s);
        ts.r = m ? __builtin_amdgcn_readlane(ts.lrad, s) : -1;
        ts.py = div_floor(qy * ts.side, q_side);
        ts.px = div_floor(qx * ts.side, q_side);
    }
    const int r = ts.r;
    if (r < 0) return 0u;
    const int local = c.base - ts.off;
    const int y0 = __builtin_amdgcn_readfirstlane(div_floor(local, ts.side));
    const int x0 = local - y0 * ts.side;
    uint32_t rows = 0u, cols = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        rows |= (uint32_t)(abs(y0 + k - ts.py) <= r) << k;
        cols |= (uint32_t)(abs(x0 + 4 * g + k - ts.px) <= r) << k;
    }
    uint32_t bits = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= ((rows >> k) & 1u) ? (cols << (4 * k)) : 0u;
    return bits;
}

// Work item -> (b h, query tile).  Kept lists differ in length (edge tiles
// of a CSLA window keep fewer key tiles than interior ones), so the launch
// ends with workgroups of long lists still running on a few slots while the
// rest of the chip idles.  The items of two consecutive heads are therefore
// interleaved and each head's query tiles taken in descending list length
// (ties by tile id): the workgroups dispatched as slots free up take the
// longest lists first.  Every workgroup ranks the counts of its head itself
// (one key per lane in LDS, count then tile id: distinct keys, a strict
// total order), so all agree on one permutation.  Heads with more than 64
// query tiles, and walks without a list, keep the natural order.
// PAIRS: the items are pairs of query tiles (2i, 2i + 1), ranked by the sum of
// their two list lengths.  Returns whether the items were ranked; then (not
// PAIRS) `count` is the list count of the chosen tile as stored, read from
// the lanes that ranked it.
template <bool PAIRS = false>
__device__ __forceinline__ bool work_tile(const AttnArgs& a, int work, int nqt, int lane, int* keys, int& bh,
                                          int& qt, int& count) {
    bh = work / nqt;
    qt = work - bh * nqt;
    if (a.kv_cnt == nullptr || nqt > 64) return false;
    const int n_bh = a.B * a.H;
    const int pair = bh >> 1;
    const int j = work - 2 * pair * nqt;               // place within the pair's items
    const bool two = 2 * pair + 1 < n_bh;
    const int head = two ? 2 * pair + (j & 1) : 2 * pair;
    const int r = two ? (j >> 1) : j;                  // wanted rank within the head
    const int32_t* cnt = a.kv_cnt + (a.per_head ? (int64_t)head * a.nqb : 0);
    // distinct keys, larger = earlier: the list length (clamped), then the lower item id
    int len = 0, raw = 0;
    if (lane < nqt) {
        if (PAIRS) {
            len = max(cnt[2 * lane], 0);
            if (2 * lane + 1 < a.nqb) len += max(cnt[2 * lane + 1], 0);
        } else {
            raw = cnt[lane];
            len = max(raw, 0);
        }
    }
    const int key = lane < nqt ? min(len, (1 << 24) - 1) * 64 + (63 - lane) : -1;
    keys[lane] = key;
    int rank = 0;
#pragma unroll
    for (int u = 0; u < 64; u += 4) {
        const int4 k4 = *(const int4*)(keys + u);
        rank += (k4.x > key) + (k4.y > key) + (k4.z > key) + (k4.w > key);
    }
    const uint64_t hit = __ballot(lane < nqt && rank == r);
    bh = head;
    qt = __builtin_ctzll(hit);
    count = __builtin_amdgcn_readlane(raw, qt);
    return true;
}

// OC: the O_cache correction of a later scale (the decision scale's full
// minus sparse output at the query's nearest-upsampled decision token) is
// added to the normalised output before its one rounding to bf16.
// MULTI: the work item is given (a launch over several targets), else taken
// from the workgroup id.
template <int D, bool DENSE, bool TOKEN, bool OC, bool MULTI = false>
__device__ __forceinline__ void attn_fwd_bf16_body(const AttnArgs& a, const int work_in = 0) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int STAGE = 32 * D * 2;
    __shared__ __attribute__((aligned(1024))) char smem[4 * STAGE];   // [stage][K, V]
    __shared__ uint2 table[DENSE ? 1 : kTableCap];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 31, g = lane >> 5;  // query column and lane half of this lane

    const int64_t nqt = DENSE ? (a.nq + 63) / 64 : a.nqb;
    const int work = MULTI ? work_in : xcd_remap(blockIdx.x, gridDim.x);
    int bh, qt;
    LaneGeom lg;
    int ranked_count = 0;
    bool ranked = false;
    if (DENSE) {
        bh = work / nqt;
        qt = work - bh * nqt;
    } else {
        lg = lane_geom(a.g, lane);   // independent of the item: in flight during the ranking
        __shared__ __attribute__((aligned(16))) int rank_keys[2][64];
        ranked = work_tile(a, work, nqt, lane, rank_keys[wave], bh, qt, ranked_count);
        bh = __builtin_amdgcn_readfirstlane(bh);
        qt = __builtin_amdgcn_readfirstlane(qt);
    }
    const int b = bh / a.H, h = bh - b * a.H;

    // ---- the query this lane holds (column n of the wave's 32 queries)
    int64_t tok;
    bool qvalid = true;
    int qy = 0, qx = 0;   // the query's grid coordinates (token mode)
    if (DENSE) {
        tok = 64 * (int64_t)qt + 32 * wave + n;
        qvalid = tok < a.nq;
        if (!qvalid) tok = a.nq - 1;
    } else {
        const int nbq = a.q_side >> 3;
        const int ti = qt / nbq, tj = qt - ti * nbq;
        qy = 8 * ti + 4 * wave + (n >> 3);
        qx = 8 * tj + (n & 7);
        tok = (int64_t)qy * a.q_side + qx;
    }
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;
    const __bf16* vh = a.v + b * a.sv_b + h * a.sv_h;
    const int32_t krb = (int32_t)(a.sk_t * 2), vrb = (int32_t)(a.sv_t * 2);
    const float c = a.scale_log2;
    const lds_ptr L = (lds_ptr)smem;
    const char* sm = smem;

    // The list count and the first 64 list entries are loaded before the Q^T
    // operands, so that waiting for the entries does not wait for Q (vector
    // loads complete in issue order); Q's loads are in flight while the walk is
    // set up.
    Walk w, w0;   // w0: the walk as it starts (for the safe pass)
    int first64 = 0;
    if (!DENSE) {
        const int64_t row = (a.per_head ? (int64_t)bh * a.nqb : 0) + qt;
        if (a.kv_cnt != nullptr) {
            w.cnt = ranked ? ranked_count : a.kv_cnt[row];
            w.idx = a.kv_idx + row * a.nkb;
        } else {   // token mode without a list: every key tile
            w.cnt = a.nkb;
            w.idx = nullptr;
        }
        first64 = lane < w.cnt ? (w.idx != nullptr ? w.idx[lane] : lane) : -1;
    }
    WaveState<D> st;
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) st.qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    init_lds_offsets<D>(st, lane);
    LoadPlan<D> plan;
    make_plan<D>(plan, wave, lane, a.sk_t, a.sv_t);

    // ---- the walk, in table builds of up to kTableCap chunks (the first one
    // before the accumulators are live)
    __shared__ int table_n;
    int nch;
    bool first_loaded = false;   // the first chunk's loads already issued
    if (DENSE) {
        w.cnext = 0;
        w.cend = (int32_t)a.nk;
        w.j = w.cnt = 0;
        w.idx = nullptr;
        nch = (w.cend + 31) >> 5;
        w0 = w;
    } else {
        // leading run of tiles 0,1,2,...: whole scales kept from the start form
        // one contiguous token range
        int p = 0;
        uint64_t off = __ballot(first64 != lane);
        while (!off) {   // runs past 64 entries (the loads of later entries are waited for in here)
            p += 64;
            const int v = (p + lane < w.cnt) ? (w.idx != nullptr ? w.idx[p + lane] : p + lane) : -1;
            off = __ballot(v != p + lane);
        }
        p += __builtin_ctzll(off);
        // scales wholly inside the run: those whose tiles all precede tile p
        int s = __popcll(__ballot(lane >= 1 && lane <= a.g.n_scales && lg.tb <= p));
        if (TOKEN) s = min(s, a.n_sink);   // only sink scales skip the token test
        w.cnext = 0;
        w.cend = __builtin_amdgcn_readlane(lg.off, s);
        w.j = __builtin_amdgcn_readlane(lg.tb, s);
        w0 = w;
        // the run's first chunk is known now: its loads overlap the table build
        if (w.cend > 0) {
            const int nv = min(32, w.cend);
            load_chunk<D>(plan, kh, vh, krb, vrb, unpack_chunk(0, pack_info(8, 4, 8, nv)), L, L + STAGE, wave,
                          lane);
            first_loaded = true;
        }
        if (wave == 0) {
            const int nb = build_table(w, a.g, lg, table, lane, first64, true);
            if (lane == 0) table_n = nb;
        }
        __syncthreads();   // table visible to both waves
        nch = __builtin_amdgcn_readfirstlane(table_n);
    }

    // The walk, in two forms.  The fast form (EXACT false) takes the running
    // maximum from a walk's first chunk and afterwards takes every chunk's
    // weights against it, raising it after a chunk whose weights sum above
    // kSumCap; a weight that overflows (a score more than 127 above the
    // running maximum, log2 domain) leaves a non-finite value, and both waves
    // then redo the walk in the exact form, which raises the maximum to each
    // chunk's before its weights.
    __shared__ int bad_flag[2];
    TokenState ts;
    auto walk = [&](auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        if (EXACT) {   // restart the walk
            w = w0;
            if (!DENSE) {
                if (wave == 0) {
                    const int nb = build_table(w, a.g, lane_geom(a.g, lane), table, lane);
                    if (lane == 0) table_n = nb;
                }
                __syncthreads();
                nch = __builtin_amdgcn_readfirstlane(table_n);
            } else {
                nch = (w.cend + 31) >> 5;
            }
        }
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] = (f32x16)0.0f;
        st.m_run = -1e30f;   // finite: a fully masked chunk gives P = 0, not NaN
        st.l_run = 0.0f;
        if (TOKEN) token_init(ts, a, lane);
        PipeState<D> ps;
        pipe_reset<D>(ps);
        auto attend = [&](auto ex_tag, const char* kst, const char* vst, const Chunk& cc) {
            pipe_chunk<D, decltype(ex_tag)::value>(st, ps, kst, vst, cc, c, lane,
                                                   TOKEN ? csla_token_bits(ts, cc, qy, qx, a.q_side, g) : 0xffffu);
        };
        int walked = 0;
        while (nch > 0) {
            walked += nch;
            // descriptors of chunks [win, win + 64) in registers, lane i = chunk win + i
            int win = 0;
            uint32_t d0 = 0, d1 = 0;
            if (!DENSE) {
                const uint2 t = table[min(lane, kTableCap - 1)];
                d0 = t.x;
                d1 = t.y;
            }
            auto desc = [&](int ci) -> Chunk {
                if (DENSE) {
                    const int base = 32 * ci;
                    return unpack_chunk(base, pack_info(8, 4, 8, min(32, w.cend - base)));
                }
                if (ci - win >= 64) {
                    win += 64;
                    const uint2 t = table[min(win + lane, kTableCap - 1)];
                    d0 = t.x;
                    d1 = t.y;
                }
                return unpack_chunk((int32_t)__builtin_amdgcn_readlane(d0, ci - win),
                                    __builtin_amdgcn_readlane(d1, ci - win));
            };

            // two LDS stages, one barrier per chunk: after it, every wave has its
            // loads of this chunk in LDS and has finished the previous chunk, whose
            // stage then takes the next prefetch
            Chunk cur = desc(0), nxt;
            if (!first_loaded) load_chunk<D>(plan, kh, vh, krb, vrb, cur, L, L + STAGE, wave, lane);
            first_loaded = false;
            // chunk ci in stage ci % 2, its successor loaded into the other;
            // chunk ci's product is taken in the step of chunk ci + 1 (or in
            // the drain after the segment's last chunk)
            auto step = [&](auto stage_tag, auto ex_tag, int ci) {
                constexpr int S = decltype(stage_tag)::value ? 1 : 0;
                // this wave's loads of chunk ci, and its V^T reads of chunk ci - 1 (whose
                // stage the loads issued below overwrite), are complete on both waves
                st.q_ready();
                wait_all();
                wg_barrier();
                if (ci + 1 < nch) {
                    nxt = desc(ci + 1);
                    load_chunk<D>(plan, kh, vh, krb, vrb, nxt, L + 2 * (1 - S) * STAGE, L + (3 - 2 * S) * STAGE,
                                  wave, lane);
                }
                attend(ex_tag, sm + 2 * S * STAGE, sm + (2 * S + 1) * STAGE, cur);
                cur = nxt;
            };
            int ci0 = 0;
            if (!EXACT && walked == nch) {   // the walk's first two chunks: the first exact
                step(IntC<false>{}, IntC<true>{}, 0);
                if (nch > 1) step(IntC<true>{}, IntC<false>{}, 1);
                ci0 = 2;
            }
            int ci = ci0;
            for (; ci + 1 < nch; ci += 2) {   // whole pairs: the loop has one exit
                step(IntC<false>{}, IntC<EXACT>{}, ci);
                step(IntC<true>{}, IntC<EXACT>{}, ci + 1);
            }
            if (ci < nch) step(IntC<false>{}, IntC<EXACT>{}, ci);
            pipe_drain<D>(st, ps);
            if (DENSE) break;
            // long lists: rebuild the table with what remains of the walk
            __syncthreads();   // every wave done with the table and the stages
            if (wave == 0) {
                const int nb = build_table(w, a.g, lane_geom(a.g, lane), table, lane);
                if (lane == 0) table_n = nb;
            }
            __syncthreads();
            nch = __builtin_amdgcn_readfirstlane(table_n);
        }
        // a non-finite value, or a zero row sum after a walk over chunks, asks
        // for the exact form
        bool bad = !(__builtin_fabsf(st.l_run) <= 3.0e38f) || (walked > 0 && half_swap_sum(st.l_run) == 0.0f);
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) bad |= !(__builtin_fabsf(st.oacc[mb][i]) <= 3.0e38f);
        return bad;
    };
    {
        const bool wbad = __builtin_amdgcn_ballot_w64(walk(IntC<false>{})) != 0;
        __syncthreads();   // every wave done with the stages and the table
        if (lane == 0) bad_flag[wave] = wbad ? 1 : 0;
        __syncthreads();
        if (bad_flag[0] | bad_flag[1]) walk(IntC<true>{});
    }

    // ---- epilogue
    const float l_tot = half_swap_sum(st.l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qvalid) {
        __bf16* op = a.o + b * a.so_b + h * a.so_h + tok * a.so_t;
        if constexpr (OC) {
            // decision token (floor(y h_D / h_q), floor(x h_D / h_q)) of query
            // (y, x); y and x recomputed from the token (below 2^30) rather than
            // kept live across the walk
            const uint32_t hq = (uint32_t)a.q_side, sd = (uint32_t)a.oc_side;
            const uint32_t y = (uint32_t)tok / hq, x = (uint32_t)tok - y * hq;
            const int64_t s = (int64_t)(y * sd / hq) * sd + x * sd / hq;
            const __bf16* fp = a.oc_full + b * a.sf_b + h * a.sf_h + s * a.sf_t;
            const __bf16* pp = a.oc_sparse + b * a.sp_b + h * a.sp_h + s * a.sp_t;
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int j = 32 * mb + 8 * kk + 4 * g;
                    const bf16x4 f = *(const bf16x4*)(fp + j);
                    const bf16x4 p = *(const bf16x4*)(pp + j);
                    bf16x4 val;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        val[e] = (__bf16)(st.oacc[mb][4 * kk + e] * inv + ((float)f[e] - (float)p[e]));
                    *(bf16x4*)(op + j) = val;
                }
            }
        } else {
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
        }
        if (a.lse != nullptr && g == 0) {
            const int64_t nq_tot = DENSE ? a.nq : (int64_t)a.q_side * a.q_side;
            a.lse[(int64_t)bh * nq_tot + tok] =
                l_tot > 0.0f ? (st.m_run + __builtin_log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
    }
}

template <int D, bool DENSE, bool TOKEN>
__global__ __launch_bounds__(128, 2) void attn_fwd_bf16_kernel(const AttnArgs a) {
    attn_fwd_bf16_body<D, DENSE, TOKEN, false>(a);
}

// Block-sparse attention of a later scale with its O_cache correction.
template <int D>
__global__ __launch_bounds__(128, 2) void attn_fwd_ocache_bf16_kernel(const AttnArgs a) {
    attn_fwd_bf16_body<D, false, false, true>(a);
}

// Block-sparse attention of several query scales over one cache in one
// launch (with or without the O_cache correction).  Each workgroup runs the
// walk of attn_fwd_bf16_kernel for one work item of one target, so every
// output is bit-identical to that target's own launch; one grid over all the
// targets fills the chip where a small scale alone would leave CUs idle and
// pay its own launch ramp and tail.  Work order: head pairs outermost (every
// target of a head attends to the same cache, so one XCD's L2 holds the K/V
// of its few heads for all of them), then the targets in the caller's order,
// then the pair's items as attn_fwd_bf16_kernel orders one target's.
template <int D, bool OC>
__global__ __launch_bounds__(128, 2) void attn_multi_bf16_kernel(const MultiAttnArgs m) {
    const int G = xcd_remap(blockIdx.x, gridDim.x);
    const int n_bh = m.t[0].B * m.t[0].H, full_pairs = n_bh >> 1;
    int sum2 = 0;
#pragma unroll
    for (int t = 0; t < kMaxAttnTargets; ++t)
        if (t < m.n_targets) sum2 += 2 * m.t[t].nqb;
    int p, r, mult;
    if (G < full_pairs * sum2) {
        p = G / sum2;
        r = G - p * sum2;
        mult = 2;
    } else {   // the last head of an odd count: a pair of one
        p = full_pairs;
        r = G - full_pairs * sum2;
        mult = 1;
    }
    int t = 0;
#pragma unroll
    for (int u = 0; u + 1 < kMaxAttnTargets; ++u) {
        if (t == u && u + 1 < m.n_targets && r >= mult * m.t[u].nqb) {
            r -= mult * m.t[u].nqb;
            t = u + 1;
        }
    }
    attn_fwd_bf16_body<D, false, false, OC, true>(m.t[t], 2 * p * m.t[t].nqb + r);
}

// Dense attention of several query sets over prefixes of one cache in one
// launch: each workgroup runs the one-pass dense walk of attn_fwd_bf16_kernel
// for one 64-query block of one target (bit-identical to a one-target launch
// that walks its blocks in one pass rather than split), so a step's many
// small dense scales cost one launch ramp and tail instead of one each.  Targets take contiguous ranges of work items in the
// caller's order.
template <int D>
__global__ __launch_bounds__(128, 2) void attn_dense_multi_bf16_kernel(const MultiDenseArgs m) {
    const int G = xcd_remap(blockIdx.x, gridDim.x);
    int t = 0;
#pragma unroll
    for (int u = 1; u < kMaxDenseTargets; ++u)
        if (u < m.n_targets && G >= m.wg_base[u]) t = u;
    AttnArgs a = m.base;
    a.q = m.q[t];
    a.o = m.o[t];
    a.lse = m.lse[t];
    a.nq = m.nq[t];
    a.nk = m.nk[t];
    a.sq_b = m.sq[t][0];
    a.sq_h = m.sq[t][1];
    a.sq_t = m.sq[t][2];
    a.so_b = m.so[t][0];
    a.so_h = m.so[t][1];
    a.so_t = m.so[t][2];
    attn_fwd_bf16_body<D, true, false, false, true>(a, G - m.wg_base[t]);
}

// ---- dense attention over few query blocks: each block's keys split over P wave pairs
//
// A dense launch over a handful of 64-query blocks (the small scales of a
// generation step, the decision scale) leaves most of the chip idle while
// every block walks all its keys in turn.  Here one workgroup = one 64-query
// block and P wave pairs: pair p walks the p-th of P contiguous ranges of
// 32-key chunks with the chunk step of attn_fwd_bf16_kernel (its own two LDS
// stages, its own running maximum, the exact first chunk and the exact redo
// of a walk that overflowed), and the pairs' maxima, row sums and O^T are
// merged through LDS at the end: the same softmax in arithmetic, summed in
// another order.  All pairs pass the same number of workgroup barriers (a
// pair with one chunk fewer passes an extra one).
template <int D, int P>
__global__ __launch_bounds__(128 * P, P == 2 ? 2 : 1) void attn_dense_split_kernel(const AttnArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int STAGE = 32 * D * 2;
    extern __shared__ __attribute__((aligned(1024))) char dyn[];   // [P][stage][K, V]; then the merge

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int part = wave >> 1, pw = wave & 1;   // wave pair, and wave within it
    const int n = lane & 31, g = lane >> 5;
    const int64_t nqt = (a.nq + 63) / 64;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = (int)(work / nqt);
    const int64_t qt = work - (int64_t)bh * nqt;
    const int b = bh / a.H, h = bh - b * a.H;
    // this lane's query (clamped for the tail block; recomputed for the epilogue
    // rather than kept live across the walk)
    auto query_tok = [&]() { return min(64 * qt + 32 * pw + n, a.nq - 1); };
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;
    const __bf16* vh = a.v + b * a.sv_b + h * a.sv_h;
    const int32_t krb = (int32_t)(a.sk_t * 2), vrb = (int32_t)(a.sv_t * 2);
    const float c = a.scale_log2;
    const lds_ptr L = (lds_ptr)(dyn + part * 4 * STAGE);   // this pair's stages (loads)

    WaveState<D> st;
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + query_tok() * a.sq_t;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) st.qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    init_lds_offsets<D>(st, lane);
    {   // the pair's stages: its offset goes into the per-lane operand offsets, so
        // that the stage constants stay in the LDS reads' immediate offsets
        const uint32_t part_off = (uint32_t)(part * 4 * STAGE);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) st.koff[s] += part_off;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.voff[mb][0] += part_off, st.voff[mb][1] += part_off;
    }
    LoadPlan<D> plan;
    make_plan<D>(plan, pw, lane, a.sk_t, a.sv_t);

    // this pair's chunks [c0, c0 + nch); nmax barriers' worth for every pair
    const int nch_all = (int)((a.nk + 31) >> 5);
    const int c0 = (int)((int64_t)nch_all * part / P);
    const int nch = (int)((int64_t)nch_all * (part + 1) / P) - c0;
    const int nmax = (nch_all + P - 1) / P;
    auto desc = [&](int ci) -> Chunk {
        const int base = 32 * (c0 + ci);
        return unpack_chunk(base, pack_info(8, 4, 8, (int)min((int64_t)32, a.nk - base)));
    };

    __shared__ int bad_any;
    auto walk = [&](auto exact_tag) {
        constexpr bool EXACT = decltype(exact_tag)::value;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] = (f32x16)0.0f;
        st.m_run = -1e30f;   // finite: a fully masked chunk gives P = 0, not NaN
        st.l_run = 0.0f;
        PipeState<D> ps;
        pipe_reset<D>(ps);
        Chunk cur = desc(0), nxt;
        if (nch > 0) load_chunk<D>(plan, kh, vh, krb, vrb, cur, L, L + STAGE, pw, lane);
        auto step = [&](auto stage_tag, auto ex_tag, int ci) {
            constexpr int S = decltype(stage_tag)::value ? 1 : 0;
            st.q_ready();
            wait_all();
            wg_barrier();
            if (ci + 1 < nch) {
                nxt = desc(ci + 1);
                load_chunk<D>(plan, kh, vh, krb, vrb, nxt, L + 2 * (1 - S) * STAGE, L + (3 - 2 * S) * STAGE, pw,
                              lane);
            }
            pipe_chunk<D, decltype(ex_tag)::value>(st, ps, dyn + 2 * S * STAGE, dyn + (2 * S + 1) * STAGE, cur, c,
                                                   lane, 0xffffu);
            cur = nxt;
        };
        int ci0 = 0;
        if (!EXACT && nch > 0) {   // the walk's first two chunks: the first exact
            step(IntC<false>{}, IntC<true>{}, 0);
            if (nch > 1) step(IntC<true>{}, IntC<false>{}, 1);
            ci0 = 2;
        }
        int ci = ci0;
        for (; ci + 1 < nch; ci += 2) {
            step(IntC<false>{}, IntC<EXACT>{}, ci);
            step(IntC<true>{}, IntC<EXACT>{}, ci + 1);
        }
        if (ci < nch) step(IntC<false>{}, IntC<EXACT>{}, ci);
        pipe_drain<D>(st, ps);
        for (int k = max(nch, 0); k < nmax; ++k) {   // the barriers of the longer pairs' last steps
            wait_all();
            wg_barrier();
        }
        bool bad = !(__builtin_fabsf(st.l_run) <= 3.0e38f) || (nch > 0 && half_swap_sum(st.l_run) == 0.0f);
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) bad |= !(__builtin_fabsf(st.oacc[mb][i]) <= 3.0e38f);
        return bad;
    };
    {
        if (threadIdx.x == 0) bad_any = 0;
        __syncthreads();
        const bool wbad = __builtin_amdgcn_ballot_w64(walk(IntC<false>{})) != 0;
        if (wbad && lane == 0) bad_any = 1;   // every writer stores the same value
        __syncthreads();   // every pair done with its stages; the flag is visible
        if (bad_any) {
            walk(IntC<true>{});
            __syncthreads();
        }
    }

    // ---- merge the pairs into pair 0 (same lane layout in every pair)
    float* mbuf = (float*)dyn;              // [P][2][64] running maxima
    float* lbuf = mbuf + P * 128;           // [P][2][64] row-sum halves
    float* obuf = lbuf + P * 128;           // [P - 1][2][MBLK * 16][64] O^T
    const int slot = (part * 2 + pw) * 64 + lane;
    if (part > 0) {
        mbuf[slot] = st.m_run;
        lbuf[slot] = st.l_run;
        float* ob = obuf + (((part - 1) * 2 + pw) * MBLK * 16) * 64 + lane;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) ob[(mb * 16 + i) * 64] = st.oacc[mb][i];
    }
    __syncthreads();
    if (part != 0) return;
    float M = st.m_run;
#pragma unroll
    for (int p = 1; p < P; ++p) M = fmaxf(M, mbuf[(p * 2 + pw) * 64 + lane]);
    {
        const float s0 = __builtin_amdgcn_exp2f(st.m_run - M);
        st.l_run *= s0;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] *= s0;
    }
#pragma unroll
    for (int p = 1; p < P; ++p) {
        const float sp = __builtin_amdgcn_exp2f(mbuf[(p * 2 + pw) * 64 + lane] - M);
        st.l_run += lbuf[(p * 2 + pw) * 64 + lane] * sp;
        const float* ob = obuf + (((p - 1) * 2 + pw) * MBLK * 16) * 64 + lane;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) st.oacc[mb][i] += ob[(mb * 16 + i) * 64] * sp;
    }
    st.m_run = M;

    // ---- epilogue (as attn_fwd_bf16_kernel's)
    const float l_tot = half_swap_sum(st.l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int64_t tok = query_tok();
    if (64 * qt + 32 * pw + n < a.nq) {
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
        if (a.lse != nullptr && g == 0)
            a.lse[(int64_t)bh * a.nq + tok] =
                l_tot > 0.0f ? (st.m_run + __builtin_log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    }
}

// ---- 128-query workgroups over pairs of query tiles (the block-128 variant)
//
// One workgroup = four waves = query tiles 2p and 2p + 1 of one (b, h)
// (128 queries; waves 0, 1 take tile 2p, waves 2, 3 tile 2p + 1, 32 queries
// each).  The chunk table walks the union of the two tiles' kept-tile lists
// (membership bitmaps in LDS), each descriptor carrying which of the two
// tiles keeps it; every chunk is loaded once for both tiles (each wave fills
// 8 of its 32 key rows) and a wave attends only to the chunks its tile keeps.
// A leading run of whole scales kept by both tiles is walked as dense
// 32-token chunks.  Per query the keys attended are exactly its tile's list;
// only the chunking of the run may differ from the 64-query kernel.
constexpr int kPairMaxNkb = kPairMaxNkbHost;    // key tiles covered by the LDS bitmaps
constexpr int kPairStages = 2;                  // LDS ring depth (K and V per stage)

template <int D>
struct PairPlan {
    static constexpr int ROWB = D * 2;          // LDS bytes per key row
    static constexpr int CH = D / 8;            // 16-byte units per row
    static constexpr int RPL = 1024 / ROWB;     // rows per wave-wide load
    static constexpr int LOADS = 8 / RPL;       // loads per wave per tensor (8 rows per wave)
    int32_t kc[LOADS], vc[LOADS];
};

template <int D>
__device__ __forceinline__ int pair_slot(int wave, int lane, int i) {
    using P = PairPlan<D>;
    return 8 * wave + i * P::RPL + lane / P::CH;            // key slot 0..31 filled by this lane
}

template <int D>
__device__ __forceinline__ void make_pair_plan(PairPlan<D>& p, int wave, int lane, int64_t sk_t, int64_t sv_t) {
    using P = PairPlan<D>;
#pragma unroll
    for (int i = 0; i < P::LOADS; ++i) {
        const int row = pair_slot<D>(wave, lane, i);
        const int unit = (lane % P::CH) ^ swz<P::CH>(row);
        p.kc[i] = (row & 7) * (int32_t)(sk_t * 2) + unit * 16;
        p.vc[i] = (row & 7) * (int32_t)(sv_t * 2) + unit * 16;
        asm volatile("" : "+v"(p.kc[i]), "+v"(p.vc[i]));
    }
}

// Wave `wave` fills key rows [8 wave, 8 wave + 8) of a stage: chunk row `wave`.
template <int D>
__device__ __forceinline__ void load_chunk_pair(const PairPlan<D>& p, const __bf16* kh, const __bf16* vh,
                                                int32_t krb, int32_t vrb, const Chunk& c, lds_ptr k_lds,
                                                lds_ptr v_lds, int wave, int lane) {
    using P = PairPlan<D>;
    if (c.full) {
        const int32_t t0 = c.base + wave * c.stride;
#pragma unroll
        for (int i = 0; i < P::LOADS; ++i) {
            const int dst = (8 * wave + i * P::RPL) * P::ROWB;
            dma16(kh, (uint32_t)(t0 * krb + p.kc[i]), k_lds + dst);
            dma16(vh, (uint32_t)(t0 * vrb + p.vc[i]), v_lds + dst);
        }
    } else {
#pragma unroll
        for (int i = 0; i < P::LOADS; ++i) {
            const int slot = pair_slot<D>(wave, lane, i);
            const int r = slot >> 3, col = slot & 7;
            const int unit16 = ((lane % P::CH) ^ swz<P::CH>(slot)) * 16;
            const bool valid = r < c.nrows && col < c.ncols && slot < c.nvalid;
            const int32_t tok = valid ? c.base + r * c.stride + col : c.base;
            const int dst = (8 * wave + i * P::RPL) * P::ROWB;
            dma16(kh, (uint32_t)(tok * krb + unit16), k_lds + dst);
            dma16(vh, (uint32_t)(tok * vrb + unit16), v_lds + dst);
        }
    }
}

// Walk state of a tile pair: the dense run [cnext, cend), then key tiles
// from `cursor` on, kept by either tile.
struct PairWalk {
    int32_t cnext, cend, cursor, nkb;
};

// Wave 0 fills the chunk table with the next descriptors of the union walk
// (bits 30, 31 of the second word: kept by the first / second tile) and
// returns how many it wrote.
__device__ __forceinline__ int build_table_pair(PairWalk& w, const DevGeom& g, uint2* table, const uint32_t* bm_a,
                                                const uint32_t* bm_b, int lane) {
    int n = 0;
    if (w.cnext < w.cend) {
        const int nc = min((w.cend - w.cnext + 31) >> 5, kTableCap);
        for (int k = lane; k < nc; k += 64) {
            const int base = w.cnext + 32 * k;
            table[k] = make_uint2((uint32_t)base, pack_info(8, 4, 8, min(32, w.cend - base)) | (3u << 30));
        }
        w.cnext = min(w.cend, w.cnext + 32 * nc);
        n = nc;
    }
    while (w.cursor < w.nkb && kTableCap - n >= 128) {
        const int id = w.cursor + lane;
        uint32_t own = 0u;
        if (id < w.nkb) own = ((bm_a[id >> 5] >> (id & 31)) & 1u) | (((bm_b[id >> 5] >> (id & 31)) & 1u) << 1);
        const bool valid = own != 0u;
        int tb = 0, side = g.side[0], off = 0, nb = g.nb[0];
        for (int s = 1; s < g.n_scales; ++s) {
            if (id >= g.tile_base[s]) {
                tb = g.tile_base[s];
                side = g.side[s];
                off = g.tok_off[s];
                nb = g.nb[s];
            }
        }
        const int local = valid ? id - tb : 0;
        int a = (int)(((float)local + 0.5f) / (float)nb);
        a -= (a * nb > local);
        a += ((a + 1) * nb <= local);
        const int b = local - a * nb, t = g.tile;
        const int rows = min(t, side - a * t), cols = min(t, side - b * t);
        const int base = off + a * t * side + b * t;
        const bool two = valid && rows > 4;
        const uint64_t vb = __ballot(valid), tb2 = __ballot(two);
        const uint64_t lt = (1ull << lane) - 1;
        const int pos = n + __popcll(vb & lt) + __popcll(tb2 & lt);
        if (valid) {
            table[pos] = make_uint2((uint32_t)base, pack_info(side, min(4, rows), cols, 32) | (own << 30));
            if (two)
                table[pos + 1] = make_uint2((uint32_t)(base + 4 * side), pack_info(side, rows - 4, cols, 32) | (own << 30));
        }
        n += __popcll(vb) + __popcll(tb2);
        w.cursor = min(w.nkb, w.cursor + 64);
    }
    return n;
}

// Leading run of a list: how many of its first entries are 0, 1, 2, ...
__device__ __forceinline__ int leading_run(const int32_t* idx, int cnt, int lane) {
    int p = 0;
    for (;;) {
        const int v = (p + lane < cnt) ? idx[p + lane] : -1;
        const uint64_t off = __ballot(v != p + lane);
        if (off) return p + __builtin_ctzll(off);
        p += 64;
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_pair_bf16_kernel(const AttnArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int MBLK = D / 32;
    constexpr int STAGE = 32 * D * 2;
    __shared__ __attribute__((aligned(1024))) char smem[2 * kPairStages * STAGE];   // [stage][K, V]
    __shared__ uint2 table[kTableCap];
    __shared__ uint32_t bm[2][kPairMaxNkb / 32];
    __shared__ int table_n, run_len[2];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 31, g = lane >> 5;
    const int tile_sel = wave >> 1, hw = wave & 1;           // which tile of the pair, which query half

    const int npair = (a.nqb + 1) >> 1;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    __shared__ __attribute__((aligned(16))) int rank_keys[4][64];
    int bh, pr;
    int unused_count;
    work_tile<true>(a, work, npair, lane, rank_keys[wave], bh, pr, unused_count);   // longest lists first
    bh = __builtin_amdgcn_readfirstlane(bh);
    pr = __builtin_amdgcn_readfirstlane(pr);
    const int b = bh / a.H, h = bh - b * a.H;
    const int qt = 2 * pr + tile_sel;
    const bool tile_ok = qt < a.nqb;                         // the pair of an odd last tile has one tile
    const int qt_c = tile_ok ? qt : a.nqb - 1;

    const int nbq = a.q_side >> 3;
    const int ti = qt_c / nbq, tj = qt_c - ti * nbq;
    const int64_t tok = (int64_t)(8 * ti + 4 * hw + (n >> 3)) * a.q_side + 8 * tj + (n & 7);
    const __bf16* kh = a.k + b * a.sk_b + h * a.sk_h;
    const __bf16* vh = a.v + b * a.sv_b + h * a.sv_h;
    const int32_t krb = (int32_t)(a.sk_t * 2), vrb = (int32_t)(a.sv_t * 2);
    const float c = a.scale_log2;
    const lds_ptr L = (lds_ptr)smem;
    const char* sm = smem;

    // ---- the two lists: membership bitmaps and the common leading run
    const int64_t row0 = (a.per_head ? (int64_t)bh * a.nqb : 0) + 2 * pr;
    const int words = (a.nkb + 31) >> 5;
    for (int i = threadIdx.x; i < 2 * (kPairMaxNkb / 32); i += 256) (&bm[0][0])[i] = 0u;
    __syncthreads();
    {
        // waves 0, 1: list of tile 2p; waves 2, 3: list of tile 2p + 1 (if any)
        const int which = wave >> 1;
        const bool has = 2 * pr + which < a.nqb;
        const int cnt = has ? min(max(a.kv_cnt[row0 + which], 0), a.nkb) : 0;
        const int32_t* idx = a.kv_idx + (row0 + which) * a.nkb;
        for (int e = (wave & 1) * 64 + lane; e < cnt; e += 128) {
            const int id = idx[e];
            if (id >= 0 && id < a.nkb) atomicOr(&bm[which][id >> 5], 1u << (id & 31));
        }
        if ((wave & 1) == 0) {
            const int p = has ? leading_run(idx, cnt, lane) : 0;
            if (lane == 0) run_len[which] = p;
        }
    }
    __syncthreads();
    PairWalk w;
    {
        const int p = min(run_len[0], run_len[1]);
        int s = 0;
        while (s < a.g.n_scales && a.g.tile_base[s + 1] <= p) ++s;
        w.cnext = 0;
        w.cend = a.g.tok_off[s];
        w.cursor = a.g.tile_base[s];
        w.nkb = a.nkb;
        (void)words;
    }
    if (wave == 0) {
        const int nb = build_table_pair(w, a.g, table, bm[0], bm[1], lane);
        if (lane == 0) table_n = nb;
    }
    __syncthreads();
    int nch = __builtin_amdgcn_readfirstlane(table_n);

    WaveState<D> st;
    const __bf16* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) st.qreg[s] = *(const bf16x8*)(qp + 16 * s + 8 * g);
    init_lds_offsets<D>(st, lane);
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) st.oacc[mb] = (f32x16)0.0f;
    st.m_run = -1e30f;
    st.l_run = 0.0f;
    PairPlan<D> plan;
    make_pair_plan<D>(plan, wave, lane, a.sk_t, a.sv_t);
    const uint32_t mine = 1u << tile_sel;

    while (nch > 0) {
        int win = 0;
        uint32_t d0, d1;
        {
            const uint2 t = table[min(lane, kTableCap - 1)];
            d0 = t.x;
            d1 = t.y;
        }
        auto desc = [&](int ci, uint32_t& own) -> Chunk {
            if (ci - win >= 64) {
                win += 64;
                const uint2 t = table[min(win + lane, kTableCap - 1)];
                d0 = t.x;
                d1 = t.y;
            }
            const uint32_t info = __builtin_amdgcn_readlane(d1, ci - win);
            own = info >> 30;
            return unpack_chunk((int32_t)__builtin_amdgcn_readlane(d0, ci - win), info);
        };
        // ring of kPairStages LDS stages, chunks loaded kPairStages - 1 ahead,
        // one barrier per chunk: after it every wave has its loads of chunk ci
        // in LDS and has finished chunk ci - 1, whose stage takes chunk
        // ci + kPairStages - 1
        constexpr int NST = kPairStages;
        constexpr int PER_CHUNK = 2 * PairPlan<D>::LOADS;       // this wave's loads per chunk (K and V)
        Chunk ring[NST];
        uint32_t own[NST];
#pragma unroll
        for (int k2 = 0; k2 < NST - 1; ++k2) {
            if (k2 < nch) {
                ring[k2] = desc(k2, own[k2]);
                load_chunk_pair<D>(plan, kh, vh, krb, vrb, ring[k2], L + 2 * k2 * STAGE, L + (2 * k2 + 1) * STAGE,
                                   wave, lane);
            }
        }
        // Q^T complete from here on: the compiler's wait for it falls here, once
        // per segment, and waits for the prefetched chunks too (issued back to
        // back, so little beyond the first), not in front of the MFMAs of every
        // chunk, where it would also wait for the loads running ahead
        st.q_ready();
        for (int ci0 = 0; ci0 < nch; ci0 += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u) {           // stage u holds chunk ci0 + u
                const int ci = ci0 + u;
                if (ci >= nch) break;
                const int ahead = min(NST - 2, nch - 1 - ci);      // chunks issued after chunk ci
                if (ahead >= 2) wait_vmcnt(2 * PER_CHUNK);
                else if (ahead == 1) wait_vmcnt(PER_CHUNK);
                else wait_vmcnt(0);
                wg_barrier();
                constexpr int dummy = 0;
                (void)dummy;
                const int nu = (u + NST - 1) % NST;                  // stage of chunk ci + NST - 1
                if (ci + NST - 1 < nch) {
                    ring[nu] = desc(ci + NST - 1, own[nu]);
                    load_chunk_pair<D>(plan, kh, vh, krb, vrb, ring[nu], L + 2 * nu * STAGE,
                                       L + (2 * nu + 1) * STAGE, wave, lane);
                }
                if (own[u] & mine) attend_chunk<D, true>(st, sm + 2 * u * STAGE, sm + (2 * u + 1) * STAGE, ring[u], c, lane);
            }
        }
        // long walks: rebuild the table with what remains
        __syncthreads();
        if (wave == 0) {
            const int nb = build_table_pair(w, a.g, table, bm[0], bm[1], lane);
            if (lane == 0) table_n = nb;
        }
        __syncthreads();
        nch = __builtin_amdgcn_readfirstlane(table_n);
    }

    // ---- epilogue (as the 64-query kernel)
    const float l_tot = half_swap_sum(st.l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (tile_ok) {
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
            const int64_t nq_tot = (int64_t)a.q_side * a.q_side;
            a.lse[(int64_t)bh * nq_tot + tok] =
                l_tot > 0.0f ? (st.m_run + __builtin_log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
        }
    }
}

hipError_t launch_attn_pair_bf16(const AttnArgs& a, int head_dim, hipStream_t stream) {
    const int64_t blocks = (int64_t)((a.nqb + 1) / 2) * a.B * a.H;
    dim3 grid((unsigned)blocks), block(256);
    if (head_dim == 128) hipLaunchKernelGGL(attn_pair_bf16_kernel<128>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(attn_pair_bf16_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

namespace {

template <auto Kernel>
hipError_t launch_dense_split(int64_t blocks, int parts, size_t shmem, const AttnArgs& a, hipStream_t stream) {
    const hipError_t e = allow_dynamic_lds<Kernel>(shmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(Kernel, dim3((unsigned)blocks), dim3(128 * parts), shmem, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_multi_bf16(const MultiAttnArgs& m, int head_dim, hipStream_t stream) {
    int64_t blocks = 0;
    for (int t = 0; t < m.n_targets; ++t) blocks += (int64_t)m.t[t].nqb * m.t[t].B * m.t[t].H;
    dim3 grid((unsigned)blocks), block(128);
    const bool oc = m.t[0].oc_full != nullptr;
    if (head_dim == 128) {
        if (oc) hipLaunchKernelGGL((attn_multi_bf16_kernel<128, true>), grid, block, 0, stream, m);
        else hipLaunchKernelGGL((attn_multi_bf16_kernel<128, false>), grid, block, 0, stream, m);
    } else {
        if (oc) hipLaunchKernelGGL((attn_multi_bf16_kernel<64, true>), grid, block, 0, stream, m);
        else hipLaunchKernelGGL((attn_multi_bf16_kernel<64, false>), grid, block, 0, stream, m);
    }
    return hipGetLastError();
}

hipError_t launch_dense_multi_bf16(const MultiDenseArgs& m, int head_dim, hipStream_t stream) {
    dim3 grid((unsigned)m.wg_base[m.n_targets]), block(128);
    if (head_dim == 128) hipLaunchKernelGGL(attn_dense_multi_bf16_kernel<128>, grid, block, 0, stream, m);
    else hipLaunchKernelGGL(attn_dense_multi_bf16_kernel<64>, grid, block, 0, stream, m);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool dense, hipStream_t stream) {
    const int64_t nqt = dense ? (a.nq + 63) / 64 : a.nqb;
    const int64_t blocks = nqt * a.B * a.H;
    dim3 grid((unsigned)blocks), block(128);
    const bool token = a.token != 0 && !dense;
    if (dense) {
        // few query blocks: split each block's keys over wave pairs so that the
        // launch still fills the chip in one round (4 pairs: 128 KB of LDS, one
        // workgroup per CU; 2 pairs: two per CU), each pair walking >= 6 chunks
        // (shorter walks lose more to the merge than they gain)
        const int64_t nch_all = (a.nk + 31) >> 5;
        const size_t stage = (size_t)32 * head_dim * 2;
        if (blocks <= 256 && nch_all >= 24) {
            if (head_dim == 128)
                return launch_dense_split<attn_dense_split_kernel<128, 4>>(blocks, 4, 4 * 4 * stage, a, stream);
            return launch_dense_split<attn_dense_split_kernel<64, 4>>(blocks, 4, 4 * 4 * stage, a, stream);
        }
        if (blocks <= 512 && nch_all >= 12) {
            if (head_dim == 128)
                return launch_dense_split<attn_dense_split_kernel<128, 2>>(blocks, 2, 2 * 4 * stage, a, stream);
            return launch_dense_split<attn_dense_split_kernel<64, 2>>(blocks, 2, 2 * 4 * stage, a, stream);
        }
    }
    const bool oc = a.oc_full != nullptr && !dense && !token;
    if (head_dim == 128) {
        if (dense) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true, false>), grid, block, 0, stream, a);
        else if (token) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false, true>), grid, block, 0, stream, a);
        else if (oc) hipLaunchKernelGGL(attn_fwd_ocache_bf16_kernel<128>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false, false>), grid, block, 0, stream, a);
    } else {
        if (dense) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true, false>), grid, block, 0, stream, a);
        else if (token) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false, true>), grid, block, 0, stream, a);
        else if (oc) hipLaunchKernelGGL(attn_fwd_ocache_bf16_kernel<64>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vs

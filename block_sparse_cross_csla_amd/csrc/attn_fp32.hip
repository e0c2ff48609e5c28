// fp32 block-sparse (and dense) attention forward.
//
// Same operation as the bf16 kernel (SparVAR, ai.info summary, "Main
// Findings": block-wise sparse attention over the kept tiles), in fp32
// throughout, for the small fp32 workload and for checking.  It is written for
// clarity rather than speed: one workgroup per query tile (up to 64 queries),
// four lanes per query each holding a quarter of the head dimension, keys
// visited one at a time with an exact online softmax.
#include "kernel_args.h"

namespace vs {

template <int D, bool DENSE>
__global__ __launch_bounds__(256) void attn_fwd_fp32_kernel(const AttnF32Args a) {
    constexpr int PART = D / 4;
    const int slot = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int64_t nqt = DENSE ? (a.nq + 63) / 64 : a.nqb;
    const int bh = blockIdx.x / nqt, qt = blockIdx.x - bh * nqt;
    const int b = bh / a.H, h = bh - b * a.H;
    const int t = a.g.tile;

    int64_t tok;
    bool active;
    if (DENSE) {
        tok = 64 * (int64_t)qt + slot;
        active = tok < a.nq;
    } else {
        const int nbq = a.q_side / t;
        const int ti = qt / nbq, tj = qt - ti * nbq;
        active = slot < t * t;
        tok = (int64_t)(ti * t + slot / t) * a.q_side + tj * t + slot % t;
    }
    if (!active) tok = 0;

    float qv[PART], ov[PART];
    const float* qp = a.q + b * a.sq_b + h * a.sq_h + tok * a.sq_t + part * PART;
#pragma unroll
    for (int i = 0; i < PART; ++i) {
        qv[i] = qp[i];
        ov[i] = 0.0f;
    }
    const float* kh = a.k + b * a.sk_b + h * a.sk_h + part * PART;
    const float* vh = a.v + b * a.sv_b + h * a.sv_h + part * PART;
    float m = -INFINITY, l = 0.0f;

    auto visit = [&](int64_t key) {
        const float* kp = kh + key * a.sk_t;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < PART; ++i) s = __builtin_fmaf(qv[i], kp[i], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        const float x = s * a.scale_log2;
        const float m_new = fmaxf(m, x);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        const float p = __builtin_amdgcn_exp2f(x - m_new);
        l = l * alpha + p;
        const float* vp = vh + key * a.sv_t;
#pragma unroll
        for (int i = 0; i < PART; ++i) ov[i] = __builtin_fmaf(p, vp[i], ov[i] * alpha);
        m = m_new;
    };

    if (DENSE) {
        for (int64_t key = 0; key < a.nk; ++key) visit(key);
    } else {
        const int64_t row = (a.per_head ? (int64_t)bh * a.nqb : 0) + qt;
        const int cnt = a.kv_cnt[row];
        const int32_t* idx = a.kv_idx + row * a.nkb;
        for (int j = 0; j < cnt; ++j) {
            const int id = min(max(idx[j], 0), a.g.tile_base[a.g.n_scales] - 1);
            const int s = scale_of_tile(a.g, id);
            const int local = id - a.g.tile_base[s];
            const int nb = a.g.nb[s], side = a.g.side[s];
            const int ta = local / nb, tb = local - ta * nb;
            const int rows = min(t, side - ta * t), cols = min(t, side - tb * t);
            for (int r = 0; r < rows; ++r)
                for (int cix = 0; cix < cols; ++cix)
                    visit(a.g.tok_off[s] + (int64_t)(ta * t + r) * side + tb * t + cix);
        }
    }

    if (active) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float* op = a.o + b * a.so_b + h * a.so_h + tok * a.so_t + part * PART;
#pragma unroll
        for (int i = 0; i < PART; ++i) op[i] = ov[i] * inv;
        if (a.lse != nullptr && part == 0) {
            const int64_t nq_tot = DENSE ? a.nq : (int64_t)a.q_side * a.q_side;
            a.lse[(int64_t)bh * nq_tot + tok] =
                l > 0.0f ? (m + __builtin_log2f(l)) * 0.6931471805599453f : -INFINITY;
        }
    }
}

hipError_t launch_attn_fp32(const AttnF32Args& a, int head_dim, bool dense, hipStream_t stream) {
    const int64_t nqt = dense ? (a.nq + 63) / 64 : a.nqb;
    dim3 grid((unsigned)(nqt * a.B * a.H)), block(256);
    if (head_dim == 128) {
        if (dense) hipLaunchKernelGGL((attn_fwd_fp32_kernel<128, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_fp32_kernel<128, false>), grid, block, 0, stream, a);
    } else {
        if (dense) hipLaunchKernelGGL((attn_fwd_fp32_kernel<64, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_fp32_kernel<64, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vs

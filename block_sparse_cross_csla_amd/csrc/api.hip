// The C ABI of libvarsparse: argument validation on the host, then kernel
// launches on the caller's stream.  Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "kernel_args.h"

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return VARSPARSE_OK;
    g_last_hip = (int)e;
    return VARSPARSE_EHIP;
}

// Geometry: 1..32 scales, positive strictly ascending sides, tile >= 1, and a
// cache small enough for 32-bit token indices.
int check_geom(const varsparse_geom* g) {
    if (g == nullptr) return VARSPARSE_EINVAL;
    if (g->n_scales < 1 || g->n_scales > VARSPARSE_MAX_SCALES || g->tile < 1) return VARSPARSE_EINVAL;
    int64_t total = 0;
    for (int s = 0; s < g->n_scales; ++s) {
        if (g->side[s] < 1 || g->side[s] > 65535) return VARSPARSE_EINVAL;
        if (s > 0 && g->side[s] <= g->side[s - 1]) return VARSPARSE_EINVAL;
        total += (int64_t)g->side[s] * g->side[s];
    }
    if (total >= (int64_t)1 << 30) return VARSPARSE_EINVAL;
    return VARSPARSE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool strides_ok(const int64_t* st, int n, int64_t unit) {
    for (int i = 0; i < n; ++i)
        if (st[i] < 0 || st[i] % unit != 0) return false;
    return true;
}

bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

// The bf16 kernels address K and V of one head with 32-bit byte offsets.
bool offsets_fit(int64_t nk, int64_t sk_t, int64_t sv_t, int head_dim) {
    const int64_t lim = (int64_t)1 << 31;
    return (nk - 1) * sk_t * 2 + head_dim * 2 < lim && (nk - 1) * sv_t * 2 + head_dim * 2 < lim;
}

constexpr double kLog2e = 1.4426950408889634;

}  // namespace

extern "C" {

int varsparse_geom_counts(const varsparse_geom* geom, int32_t q_scale, int32_t* nqb, int32_t* nkb,
                          int64_t* nq, int64_t* nk) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    const vs::DevGeom d = vs::make_dev_geom(*geom, q_scale);
    if (nqb) *nqb = d.nb[q_scale] * d.nb[q_scale];
    if (nkb) *nkb = d.tile_base[q_scale + 1];
    if (nq) *nq = (int64_t)geom->side[q_scale] * geom->side[q_scale];
    if (nk) *nk = d.tok_off[q_scale + 1];
    return VARSPARSE_OK;
}

int varsparse_window_radius(int32_t n_scales, int32_t q_scale, const int32_t* windows, int32_t n_windows,
                            int32_t* radius) {
    if (n_scales < 1 || n_scales > VARSPARSE_MAX_SCALES || windows == nullptr || radius == nullptr)
        return VARSPARSE_EINVAL;
    if (n_windows < 1 || n_windows > n_scales) return VARSPARSE_EINVAL;
    const int first = n_scales - n_windows;
    if (q_scale < first || q_scale >= n_scales) return VARSPARSE_EINVAL;
    const int w = windows[q_scale - first];
    if (w < 1 || w % 2 == 0) return VARSPARSE_EINVAL;
    for (int s = 0; s <= q_scale; ++s) radius[s] = (w - 1) / 2;
    return VARSPARSE_OK;
}

int varsparse_build_mask(const varsparse_geom* geom, int32_t q_scale, int32_t n_sink, const int32_t* radius,
                         int32_t budget, uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx, void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (n_sink < 0 || n_sink > q_scale) return VARSPARSE_EINVAL;
    if (kv_cnt == nullptr || kv_idx == nullptr) return VARSPARSE_EINVAL;
    if (budget == 0 || budget < -1) return VARSPARSE_EINVAL;
    if (budget == -1 && radius == nullptr) return VARSPARSE_EINVAL;
    vs::MaskArgs a{};
    a.g = vs::make_dev_geom(*geom, q_scale);
    a.q_scale = q_scale;
    a.n_sink = n_sink;
    a.budget = budget;
    a.nkb = a.g.tile_base[q_scale + 1];
    if (budget > 0 && a.nkb > 4096) return VARSPARSE_EUNSUPPORTED;
    const int sink_tiles = a.g.tile_base[n_sink];
    a.keep_n = budget > 0 ? (int)std::min<int64_t>(a.nkb, std::max<int64_t>(budget, sink_tiles + 1)) : 0;
    for (int s = 0; s <= q_scale; ++s) a.radius[s] = budget == -1 ? radius[s] : -1;
    a.mask = mask;
    a.kv_cnt = kv_cnt;
    a.kv_idx = kv_idx;
    const int nqb = a.g.nb[q_scale] * a.g.nb[q_scale];
    return hip_status(vs::launch_csla_mask(a, nqb, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// CS4A with selection rule 0 (top-p, param = p) or 1 (Top-K fraction).
int map_indices_impl(const varsparse_geom* geom, int32_t d_scale, int32_t n_targets, const int32_t* t_scales,
                     int32_t n_sink, int rule, float top_p, varsparse_dtype dtype, int32_t B, int32_t H,
                     int32_t head_dim, const void* q_d, const int64_t q_strides[3], const void* k,
                     const int64_t k_strides[3], float softmax_scale, float* scores,
                     int32_t* sel_cnt, int32_t* sel_idx, int32_t* const* kv_cnt, int32_t* const* kv_idx,
                     void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (n_targets < 1 || n_targets > vs::kMaxTargets || t_scales == nullptr) return VARSPARSE_EINVAL;
    if (kv_cnt == nullptr || kv_idx == nullptr) return VARSPARSE_EINVAL;
    if (d_scale < 0 || d_scale >= geom->n_scales || geom->side[d_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    const bool empty = B == 0 || H == 0;
    int t_max = d_scale;
    for (int i = 0; i < n_targets; ++i) {
        const int T = t_scales[i];
        if (T < d_scale || T >= geom->n_scales || geom->side[T] % geom->tile != 0) return VARSPARSE_EINVAL;
        if (!empty && (kv_cnt[i] == nullptr || kv_idx[i] == nullptr)) return VARSPARSE_EINVAL;
        t_max = std::max(t_max, T);
    }
    if (n_sink < 0 || n_sink > d_scale) return VARSPARSE_EINVAL;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return VARSPARSE_EINVAL;
    if (empty) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (scores == nullptr) return VARSPARSE_EINVAL;
    if ((sel_cnt == nullptr) != (sel_idx == nullptr)) return VARSPARSE_EINVAL;
    const vs::DevGeom gD = vs::make_dev_geom(*geom, d_scale);
    const vs::DevGeom gT = vs::make_dev_geom(*geom, t_max);
    const int nqbD = gD.nb[d_scale] * gD.nb[d_scale], nkbD = gD.tile_base[d_scale + 1];
    if (nkbD > 240) return VARSPARSE_EUNSUPPORTED;
    vs::SelMapArgs m{};
    m.n_targets = n_targets;
    int64_t groups = 0;
    for (int i = 0; i < n_targets; ++i) {
        const int T = t_scales[i];
        m.t_scale[i] = T;
        m.nqbT[i] = gT.nb[T] * gT.nb[T];
        m.nkbT[i] = gT.tile_base[T + 1];
        m.group_base[i] = (int32_t)groups;
        m.kv_cnt[i] = kv_cnt[i];
        m.kv_idx[i] = kv_idx[i];
        groups += (m.nqbT[i] + 3) / 4;
    }
    m.group_base[n_targets] = (int32_t)groups;
    if ((int64_t)B * H * std::max<int64_t>(nqbD, groups) > 0x7fffffff) return VARSPARSE_EINVAL;
    m.groups_total = (int32_t)groups;
    if (q_d != nullptr) {
        if (dtype != VARSPARSE_BF16) return VARSPARSE_EUNSUPPORTED;
        if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
        if (geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
        if (k == nullptr || q_strides == nullptr || k_strides == nullptr) return VARSPARSE_EINVAL;
        if (!aligned16(q_d) || !aligned16(k)) return VARSPARSE_EINVAL;
        if (!strides_ok(q_strides, 3, 8) || !strides_ok(k_strides, 3, 8)) return VARSPARSE_EINVAL;
        if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
        vs::ScoreArgs sa{};
        sa.q = (const __bf16*)q_d;
        sa.k = (const __bf16*)k;
        sa.scores = scores;
        sa.sq_b = q_strides[0]; sa.sq_h = q_strides[1]; sa.sq_t = q_strides[2];
        sa.sk_b = k_strides[0]; sa.sk_h = k_strides[1]; sa.sk_t = k_strides[2];
        sa.B = B;
        sa.H = H;
        sa.scale_log2 = (float)(softmax_scale * kLog2e);
        sa.d_side = geom->side[d_scale];
        sa.nqb = nqbD;
        sa.nkb = nkbD;
        sa.g = gD;
        rc = hip_status(vs::launch_cs4a_score(sa, head_dim, (hipStream_t)stream));
        if (rc) return rc;
    }
    m.g = gT;
    m.d_scale = d_scale;
    m.n_sink = n_sink;
    m.nqbD = nqbD;
    m.nkbD = nkbD;
    m.words = (nkbD + 31) / 32;
    m.rule = rule;
    // Top-K: ceil of the float32 product frac * nkb_D, clamped to [1, nkb_D]
    m.k_keep = std::min(std::max((int)ceilf(top_p * (float)nkbD), 1), nkbD);
    m.top_p = (double)top_p;
    m.scores = scores;
    m.sel_cnt = sel_cnt;
    m.sel_idx = sel_idx;
    return hip_status(vs::launch_cs4a_select_map(m, B * H, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int varsparse_map_indices(const varsparse_geom* geom, int32_t d_scale, int32_t t_scale, int32_t n_sink,
                          float top_p, varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim,
                          const void* q_d, const int64_t q_strides[3], const void* k,
                          const int64_t k_strides[3], float softmax_scale, float* scores,
                          int32_t* sel_cnt, int32_t* sel_idx, int32_t* kv_cnt, int32_t* kv_idx,
                          void* stream) {
    return map_indices_impl(geom, d_scale, 1, &t_scale, n_sink, 0, top_p, dtype, B, H, head_dim, q_d, q_strides,
                            k, k_strides, softmax_scale, scores, sel_cnt, sel_idx, &kv_cnt, &kv_idx, stream);
}

int varsparse_map_indices_topk(const varsparse_geom* geom, int32_t d_scale, int32_t t_scale, int32_t n_sink,
                               float top_k_frac, varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim,
                               const void* q_d, const int64_t q_strides[3], const void* k,
                               const int64_t k_strides[3], float softmax_scale, float* scores,
                               int32_t* sel_cnt, int32_t* sel_idx, int32_t* kv_cnt, int32_t* kv_idx,
                               void* stream) {
    return map_indices_impl(geom, d_scale, 1, &t_scale, n_sink, 1, top_k_frac, dtype, B, H, head_dim, q_d,
                            q_strides, k, k_strides, softmax_scale, scores, sel_cnt, sel_idx, &kv_cnt, &kv_idx,
                            stream);
}

int varsparse_map_indices_multi(const varsparse_geom* geom, int32_t d_scale, int32_t n_targets,
                                const int32_t* t_scales, int32_t n_sink, int32_t rule, float param,
                                varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim,
                                const void* q_d, const int64_t q_strides[3], const void* k,
                                const int64_t k_strides[3], float softmax_scale, float* scores,
                                int32_t* const* kv_cnt, int32_t* const* kv_idx, void* stream) {
    if (rule != VARSPARSE_SELECT_TOP_P && rule != VARSPARSE_SELECT_TOP_K) return VARSPARSE_EINVAL;
    return map_indices_impl(geom, d_scale, n_targets, t_scales, n_sink, rule, param, dtype, B, H, head_dim, q_d,
                            q_strides, k, k_strides, softmax_scale, scores, nullptr, nullptr, kv_cnt, kv_idx,
                            stream);
}

int varsparse_attn_fwd(const varsparse_geom* geom, int32_t q_scale, varsparse_dtype dtype, int32_t B, int32_t H,
                       int32_t head_dim, const void* q, const void* k, const void* v, void* o, float* lse,
                       const int64_t strides[12], float softmax_scale, const int32_t* kv_cnt,
                       const int32_t* kv_idx, int32_t lists_per_head, void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (dtype != VARSPARSE_BF16 && dtype != VARSPARSE_FP32) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    if (lists_per_head != 0 && lists_per_head != 1) return VARSPARSE_EINVAL;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (dtype == VARSPARSE_BF16 && geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
    if (dtype == VARSPARSE_FP32 && geom->tile * geom->tile > 64) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !k || !v || !o || !strides || !kv_cnt || !kv_idx) return VARSPARSE_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 12, dtype == VARSPARSE_BF16 ? 8 : 4)) return VARSPARSE_EINVAL;
    const vs::DevGeom g = vs::make_dev_geom(*geom, q_scale);
    const int nqb = g.nb[q_scale] * g.nb[q_scale];
    if ((int64_t)nqb * B * H > 0x7fffffff) return VARSPARSE_EINVAL;
    const float sl2 = (float)(softmax_scale * kLog2e);
    if (dtype == VARSPARSE_BF16) {
        if (!offsets_fit(g.tok_off[q_scale + 1], strides[5], strides[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
        vs::AttnArgs a{};
        a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o; a.lse = lse;
        a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
        a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
        a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
        a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
        a.B = B; a.H = H; a.scale_log2 = sl2;
        a.kv_cnt = kv_cnt; a.kv_idx = kv_idx; a.per_head = lists_per_head;
        a.nqb = nqb; a.nkb = g.tile_base[q_scale + 1]; a.q_side = geom->side[q_scale]; a.g = g;
        return hip_status(vs::launch_attn_bf16(a, head_dim, false, (hipStream_t)stream));
    }
    vs::AttnF32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.o = (float*)o; a.lse = lse;
    a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
    a.B = B; a.H = H; a.scale_log2 = sl2;
    a.kv_cnt = kv_cnt; a.kv_idx = kv_idx; a.per_head = lists_per_head;
    a.nqb = nqb; a.nkb = g.tile_base[q_scale + 1]; a.q_side = geom->side[q_scale]; a.g = g;
    return hip_status(vs::launch_attn_fp32(a, head_dim, false, (hipStream_t)stream));
}

int varsparse_attn_fwd_ocache(const varsparse_geom* geom, int32_t q_scale, int32_t d_scale, int32_t B, int32_t H,
                              int32_t head_dim, const void* q, const void* k, const void* v, void* o, float* lse,
                              const int64_t strides[12], float softmax_scale, const int32_t* kv_cnt,
                              const int32_t* kv_idx, int32_t lists_per_head, const void* o_full_d,
                              const void* o_sparse_d, const int64_t d_strides[6], void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (d_scale < 0 || d_scale > q_scale) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    if (lists_per_head != 0 && lists_per_head != 1) return VARSPARSE_EINVAL;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !k || !v || !o || !strides || !kv_cnt || !kv_idx) return VARSPARSE_EINVAL;
    if (!o_full_d || !o_sparse_d || !d_strides) return VARSPARSE_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VARSPARSE_EINVAL;
    if (!aligned16(o_full_d) || !aligned16(o_sparse_d)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 12, 8) || !strides_ok(d_strides, 6, 8)) return VARSPARSE_EINVAL;
    const vs::DevGeom g = vs::make_dev_geom(*geom, q_scale);
    const int nqb = g.nb[q_scale] * g.nb[q_scale];
    if ((int64_t)nqb * B * H > 0x7fffffff) return VARSPARSE_EINVAL;
    if (!offsets_fit(g.tok_off[q_scale + 1], strides[5], strides[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
    vs::AttnArgs a{};
    a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o; a.lse = lse;
    a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
    a.B = B; a.H = H; a.scale_log2 = (float)(softmax_scale * kLog2e);
    a.kv_cnt = kv_cnt; a.kv_idx = kv_idx; a.per_head = lists_per_head;
    a.nqb = nqb; a.nkb = g.tile_base[q_scale + 1]; a.q_side = geom->side[q_scale]; a.g = g;
    a.oc_full = (const __bf16*)o_full_d; a.oc_sparse = (const __bf16*)o_sparse_d;
    a.sf_b = d_strides[0]; a.sf_h = d_strides[1]; a.sf_t = d_strides[2];
    a.sp_b = d_strides[3]; a.sp_h = d_strides[4]; a.sp_t = d_strides[5];
    a.oc_side = geom->side[d_scale];
    return hip_status(vs::launch_attn_bf16(a, head_dim, false, (hipStream_t)stream));
}

int varsparse_attn_fwd_multi(const varsparse_geom* geom, int32_t n_targets, const int32_t* q_scales, int32_t B,
                             int32_t H, int32_t head_dim, const void* const* q, const void* k, const void* v,
                             void* const* o, float* const* lse, const int64_t* strides, float softmax_scale,
                             const int32_t* const* kv_cnt, const int32_t* const* kv_idx, int32_t lists_per_head,
                             int32_t d_scale, const void* o_full_d, const void* o_sparse_d,
                             const int64_t d_strides[6], void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (n_targets < 1 || n_targets > VARSPARSE_MAX_ATTN_TARGETS || !q_scales) return VARSPARSE_EINVAL;
    const bool oc = o_full_d != nullptr || o_sparse_d != nullptr;
    for (int i = 0; i < n_targets; ++i) {
        const int t = q_scales[i];
        if (t < 0 || t >= geom->n_scales || geom->side[t] % geom->tile != 0) return VARSPARSE_EINVAL;
        if (oc && (d_scale < 0 || d_scale > t)) return VARSPARSE_EINVAL;
    }
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    if (lists_per_head != 0 && lists_per_head != 1) return VARSPARSE_EINVAL;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !o || !k || !v || !strides || !kv_cnt || !kv_idx) return VARSPARSE_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return VARSPARSE_EINVAL;
    if (oc) {
        if (!o_full_d || !o_sparse_d || !d_strides) return VARSPARSE_EINVAL;
        if (!aligned16(o_full_d) || !aligned16(o_sparse_d) || !strides_ok(d_strides, 6, 8)) return VARSPARSE_EINVAL;
    }
    int64_t blocks = 0;
    vs::MultiAttnArgs m{};
    m.n_targets = n_targets;
    for (int i = 0; i < n_targets; ++i) {
        const int t = q_scales[i];
        const int64_t* st = strides + 12 * i;
        if (!q[i] || !o[i] || !kv_cnt[i] || !kv_idx[i]) return VARSPARSE_EINVAL;
        if (!aligned16(q[i]) || !aligned16(o[i])) return VARSPARSE_EINVAL;
        if (!strides_ok(st, 12, 8)) return VARSPARSE_EINVAL;
        for (int j = 3; j < 9; ++j)   // one cache: every target reads K and V alike
            if (st[j] != strides[j]) return VARSPARSE_EINVAL;
        const vs::DevGeom g = vs::make_dev_geom(*geom, t);
        const int nqb = g.nb[t] * g.nb[t];
        if (!offsets_fit(g.tok_off[t + 1], st[5], st[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
        blocks += (int64_t)nqb * B * H;
        vs::AttnArgs& a = m.t[i];
        a.q = (const __bf16*)q[i]; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o[i];
        a.lse = lse != nullptr ? lse[i] : nullptr;
        a.sq_b = st[0]; a.sq_h = st[1]; a.sq_t = st[2];
        a.sk_b = st[3]; a.sk_h = st[4]; a.sk_t = st[5];
        a.sv_b = st[6]; a.sv_h = st[7]; a.sv_t = st[8];
        a.so_b = st[9]; a.so_h = st[10]; a.so_t = st[11];
        a.B = B; a.H = H; a.scale_log2 = (float)(softmax_scale * kLog2e);
        a.kv_cnt = kv_cnt[i]; a.kv_idx = kv_idx[i]; a.per_head = lists_per_head;
        a.nqb = nqb; a.nkb = g.tile_base[t + 1]; a.q_side = geom->side[t]; a.g = g;
        if (oc) {
            a.oc_full = (const __bf16*)o_full_d; a.oc_sparse = (const __bf16*)o_sparse_d;
            a.sf_b = d_strides[0]; a.sf_h = d_strides[1]; a.sf_t = d_strides[2];
            a.sp_b = d_strides[3]; a.sp_h = d_strides[4]; a.sp_t = d_strides[5];
            a.oc_side = geom->side[d_scale];
        }
    }
    if (blocks > 0x7fffffff) return VARSPARSE_EINVAL;
    return hip_status(vs::launch_attn_multi_bf16(m, head_dim, (hipStream_t)stream));
}

int varsparse_attn_fwd_pair(const varsparse_geom* geom, int32_t q_scale, int32_t B, int32_t H, int32_t head_dim,
                            const void* q, const void* k, const void* v, void* o, float* lse,
                            const int64_t strides[12], float softmax_scale, const int32_t* kv_cnt,
                            const int32_t* kv_idx, int32_t lists_per_head, void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    if (lists_per_head != 0 && lists_per_head != 1) return VARSPARSE_EINVAL;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !k || !v || !o || !strides || !kv_cnt || !kv_idx) return VARSPARSE_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 12, 8)) return VARSPARSE_EINVAL;
    const vs::DevGeom g = vs::make_dev_geom(*geom, q_scale);
    const int nqb = g.nb[q_scale] * g.nb[q_scale];
    if ((int64_t)((nqb + 1) / 2) * B * H > 0x7fffffff) return VARSPARSE_EINVAL;
    if (g.tile_base[q_scale + 1] > vs::kPairMaxNkbHost) return VARSPARSE_EUNSUPPORTED;
    if (!offsets_fit(g.tok_off[q_scale + 1], strides[5], strides[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
    vs::AttnArgs a{};
    a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o; a.lse = lse;
    a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
    a.B = B; a.H = H; a.scale_log2 = (float)(softmax_scale * kLog2e);
    a.kv_cnt = kv_cnt; a.kv_idx = kv_idx; a.per_head = lists_per_head;
    a.nqb = nqb; a.nkb = g.tile_base[q_scale + 1]; a.q_side = geom->side[q_scale]; a.g = g;
    return hip_status(vs::launch_attn_pair_bf16(a, head_dim, (hipStream_t)stream));
}

int varsparse_attn_fwd_token(const varsparse_geom* geom, int32_t q_scale, int32_t n_sink, const int32_t* radius,
                             int32_t B, int32_t H, int32_t head_dim,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int64_t strides[12], float softmax_scale,
                             const int32_t* kv_cnt, const int32_t* kv_idx, int32_t lists_per_head, void* stream) {
    int rc = check_geom(geom);
    if (rc) return rc;
    if (q_scale < 0 || q_scale >= geom->n_scales) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] % geom->tile != 0) return VARSPARSE_EINVAL;
    if (n_sink < 0 || n_sink > q_scale || radius == nullptr) return VARSPARSE_EINVAL;
    if (geom->side[q_scale] > 4096) return VARSPARSE_EUNSUPPORTED;   // projections use 24-bit exact quotients
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    if (lists_per_head != 0 && lists_per_head != 1) return VARSPARSE_EINVAL;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (geom->tile != 8) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !k || !v || !o || !strides) return VARSPARSE_EINVAL;
    if ((kv_cnt == nullptr) != (kv_idx == nullptr)) return VARSPARSE_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 12, 8)) return VARSPARSE_EINVAL;
    const vs::DevGeom g = vs::make_dev_geom(*geom, q_scale);
    const int nqb = g.nb[q_scale] * g.nb[q_scale];
    if ((int64_t)nqb * B * H > 0x7fffffff) return VARSPARSE_EINVAL;
    if (!offsets_fit(g.tok_off[q_scale + 1], strides[5], strides[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
    vs::AttnArgs a{};
    a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o; a.lse = lse;
    a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
    a.B = B; a.H = H; a.scale_log2 = (float)(softmax_scale * kLog2e);
    a.kv_cnt = kv_cnt; a.kv_idx = kv_idx; a.per_head = kv_cnt ? lists_per_head : 0;
    a.nqb = nqb; a.nkb = g.tile_base[q_scale + 1]; a.q_side = geom->side[q_scale]; a.g = g;
    a.token = 1; a.n_sink = n_sink;
    for (int s = 0; s <= q_scale; ++s) a.radius[s] = radius[s];
    return hip_status(vs::launch_attn_bf16(a, head_dim, false, (hipStream_t)stream));
}

int varsparse_dense_attn_fwd(varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim, int64_t nq, int64_t nk,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int64_t strides[12], float softmax_scale, void* stream) {
    if (dtype != VARSPARSE_BF16 && dtype != VARSPARSE_FP32) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0 || nq < 0 || nk < 1) return VARSPARSE_EINVAL;
    if (nk >= ((int64_t)1 << 30)) return VARSPARSE_EUNSUPPORTED;
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0 || nq == 0) return VARSPARSE_OK;   // no queries: nothing to compute
    if (!q || !k || !v || !o || !strides) return VARSPARSE_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 12, dtype == VARSPARSE_BF16 ? 8 : 4)) return VARSPARSE_EINVAL;
    if (((nq + 63) / 64) * B * H > 0x7fffffff) return VARSPARSE_EINVAL;
    const float sl2 = (float)(softmax_scale * kLog2e);
    if (dtype == VARSPARSE_BF16) {
        if (!offsets_fit(nk, strides[5], strides[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
        vs::AttnArgs a{};
        a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v; a.o = (__bf16*)o; a.lse = lse;
        a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
        a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
        a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
        a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
        a.B = B; a.H = H; a.scale_log2 = sl2; a.nq = nq; a.nk = nk;
        return hip_status(vs::launch_attn_bf16(a, head_dim, true, (hipStream_t)stream));
    }
    vs::AttnF32Args a{};
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.o = (float*)o; a.lse = lse;
    a.sq_b = strides[0]; a.sq_h = strides[1]; a.sq_t = strides[2];
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.so_b = strides[9]; a.so_h = strides[10]; a.so_t = strides[11];
    a.B = B; a.H = H; a.scale_log2 = sl2; a.nq = nq; a.nk = nk;
    a.g.tile = 8;
    return hip_status(vs::launch_attn_fp32(a, head_dim, true, (hipStream_t)stream));
}

int varsparse_dense_attn_fwd_multi(int32_t n_targets, int32_t B, int32_t H, int32_t head_dim, const int64_t* nq,
                                   const int64_t* nk, const void* const* q, const void* k, const void* v,
                                   void* const* o, float* const* lse, const int64_t* strides, float softmax_scale,
                                   void* stream) {
    if (n_targets < 1 || n_targets > VARSPARSE_MAX_DENSE_TARGETS || !nq || !nk) return VARSPARSE_EINVAL;
    if (B < 0 || H < 0) return VARSPARSE_EINVAL;
    for (int i = 0; i < n_targets; ++i) {
        if (nq[i] < 0 || nk[i] < 1) return VARSPARSE_EINVAL;
        if (nk[i] >= ((int64_t)1 << 30)) return VARSPARSE_EUNSUPPORTED;
    }
    if (!scale_ok(softmax_scale)) return VARSPARSE_EINVAL;
    if (head_dim != 64 && head_dim != 128) return VARSPARSE_EUNSUPPORTED;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!q || !o || !k || !v || !strides) return VARSPARSE_EINVAL;
    if (!aligned16(k) || !aligned16(v)) return VARSPARSE_EINVAL;
    vs::MultiDenseArgs m{};
    vs::AttnArgs& a = m.base;
    a.k = (const __bf16*)k; a.v = (const __bf16*)v;
    a.sk_b = strides[3]; a.sk_h = strides[4]; a.sk_t = strides[5];
    a.sv_b = strides[6]; a.sv_h = strides[7]; a.sv_t = strides[8];
    a.B = B; a.H = H; a.scale_log2 = (float)(softmax_scale * kLog2e);
    int64_t blocks = 0;
    int n = 0;   // targets with queries
    for (int i = 0; i < n_targets; ++i) {
        const int64_t* st = strides + 12 * i;
        if (!strides_ok(st, 12, 8)) return VARSPARSE_EINVAL;
        for (int j = 3; j < 9; ++j)   // one cache: every target reads K and V alike
            if (st[j] != strides[j]) return VARSPARSE_EINVAL;
        if (!offsets_fit(nk[i], st[5], st[8], head_dim)) return VARSPARSE_EUNSUPPORTED;
        if (nq[i] == 0) continue;
        if (!q[i] || !o[i] || !aligned16(q[i]) || !aligned16(o[i])) return VARSPARSE_EINVAL;
        m.wg_base[n] = (int32_t)std::min<int64_t>(blocks, 0x7fffffff);
        blocks += ((nq[i] + 63) / 64) * B * H;
        m.q[n] = (const __bf16*)q[i]; m.o[n] = (__bf16*)o[i]; m.lse[n] = lse != nullptr ? lse[i] : nullptr;
        m.nq[n] = nq[i]; m.nk[n] = nk[i];
        for (int j = 0; j < 3; ++j) {
            m.sq[n][j] = st[j];
            m.so[n][j] = st[9 + j];
        }
        ++n;
    }
    if (blocks > 0x7fffffff) return VARSPARSE_EINVAL;
    if (n == 0) return VARSPARSE_OK;   // no queries: nothing to compute
    m.n_targets = n;
    m.wg_base[n] = (int32_t)blocks;
    return hip_status(vs::launch_dense_multi_bf16(m, head_dim, (hipStream_t)stream));
}

int varsparse_ocache_correct(int32_t B, int32_t H, int32_t head_dim, int32_t side_d, int32_t side_t,
                             const void* o_full_d, const void* o_sparse_d, void* o_t,
                             const int64_t strides[9], void* stream) {
    if (B < 0 || H < 0 || side_d < 1 || side_t < side_d || side_t > 65535) return VARSPARSE_EINVAL;
    if (head_dim < 8 || head_dim % 8 != 0 || head_dim > 1024) return VARSPARSE_EINVAL;
    if (B == 0 || H == 0) return VARSPARSE_OK;   // empty batch: nothing to compute
    if (!o_full_d || !o_sparse_d || !o_t || !strides) return VARSPARSE_EINVAL;
    if (!aligned16(o_full_d) || !aligned16(o_sparse_d) || !aligned16(o_t)) return VARSPARSE_EINVAL;
    if (!strides_ok(strides, 9, 8)) return VARSPARSE_EINVAL;
    if ((int64_t)B * H > 65535) return VARSPARSE_EUNSUPPORTED;
    vs::OcacheArgs a{};
    a.o_full = (const __bf16*)o_full_d; a.o_sparse = (const __bf16*)o_sparse_d; a.o_t = (__bf16*)o_t;
    a.sf_b = strides[0]; a.sf_h = strides[1]; a.sf_t = strides[2];
    a.sp_b = strides[3]; a.sp_h = strides[4]; a.sp_t = strides[5];
    a.so_b = strides[6]; a.so_h = strides[7]; a.so_t = strides[8];
    a.B = B; a.H = H; a.head_dim = head_dim; a.side_d = side_d; a.side_t = side_t;
    return hip_status(vs::launch_ocache_correct(a, (hipStream_t)stream));
}

int varsparse_join_lists(int32_t sets, int32_t rows, int32_t nkb, int32_t join,
                         const int32_t* a_cnt, const int32_t* a_idx, int32_t a_per_set,
                         const int32_t* b_cnt, const int32_t* b_idx, int32_t b_per_set,
                         int32_t* out_cnt, int32_t* out_idx, void* stream) {
    if (sets < 0 || rows < 1 || nkb < 1 || nkb > 65536) return VARSPARSE_EINVAL;
    if (join != VARSPARSE_JOIN_UNION && join != VARSPARSE_JOIN_INTERSECTION) return VARSPARSE_EINVAL;
    if (sets == 0) return VARSPARSE_OK;   // no list sets: nothing to compute
    if ((int64_t)sets * rows >= ((int64_t)1 << 31)) return VARSPARSE_EINVAL;
    if (!a_cnt || !a_idx || !b_cnt || !b_idx || !out_cnt || !out_idx) return VARSPARSE_EINVAL;
    if (out_cnt == a_cnt || out_cnt == b_cnt || out_idx == a_idx || out_idx == b_idx) return VARSPARSE_EINVAL;
    vs::JoinArgs g{};
    g.a_cnt = a_cnt; g.a_idx = a_idx; g.b_cnt = b_cnt; g.b_idx = b_idx;
    g.out_cnt = out_cnt; g.out_idx = out_idx;
    g.sets = sets; g.rows = rows; g.nkb = nkb; g.words = (nkb + 31) / 32; g.join = join;
    g.a_per_set = a_per_set != 0; g.b_per_set = b_per_set != 0;
    return hip_status(vs::launch_join_lists(g, (hipStream_t)stream));
}

const char* varsparse_strerror(int code) {
    switch (code) {
        case VARSPARSE_OK: return "ok";
        case VARSPARSE_EINVAL: return "invalid argument";
        case VARSPARSE_EUNSUPPORTED: return "unsupported configuration";
        case VARSPARSE_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int varsparse_last_hip_error(void) { return g_last_hip; }

}  // extern "C"

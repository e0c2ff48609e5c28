// Kernel argument blocks (passed by value) and launchers of libvarsparse.
#pragma once

#include "common.h"

namespace vs {

struct AttnArgs {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    __bf16* o;
    float* lse;
    int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
    int32_t B, H;
    float scale_log2;        // softmax_scale * log2(e)
    // block-sparse walk
    const int32_t* kv_cnt;
    const int32_t* kv_idx;
    int32_t per_head;
    int32_t nqb, nkb;
    int32_t q_side;
    DevGeom g;
    // token-exact mode (CSLA token mask inside the kept tiles; no list = every tile)
    int32_t token, n_sink;
    int32_t radius[kMaxScales];
    // dense walk
    int64_t nq, nk;
    // O_cache correction in the epilogue: decision-scale full and sparse outputs
    const __bf16* oc_full;
    const __bf16* oc_sparse;
    int64_t sf_b, sf_h, sf_t, sp_b, sp_h, sp_t;
    int32_t oc_side;
};

// Several query scales of one cache in one attention launch: per target the
// arguments of its own launch (the K / V pointers and strides, B, H, the
// scale and the O_cache inputs alike in all).
constexpr int kMaxAttnTargets = VARSPARSE_MAX_ATTN_TARGETS;   // three argument blocks fit the kernarg space

struct MultiAttnArgs {
    AttnArgs t[kMaxAttnTargets];
    int32_t n_targets;
};
static_assert(sizeof(MultiAttnArgs) <= 3072, "kernel arguments stay well inside the 4 KB kernarg space");

// Dense attention of several query sets over prefixes of one cache in one
// launch (the small scales of a generation step, each over the cache of the
// scales up to its own): per target its queries, outputs and lengths.
constexpr int kMaxDenseTargets = VARSPARSE_MAX_DENSE_TARGETS;

struct MultiDenseArgs {
    AttnArgs base;    // k, v and their strides, B, H, the scale
    int32_t n_targets;
    int32_t wg_base[kMaxDenseTargets + 1];   // first workgroup of each target (prefix sums)
    const __bf16* q[kMaxDenseTargets];
    __bf16* o[kMaxDenseTargets];
    float* lse[kMaxDenseTargets];
    int64_t nq[kMaxDenseTargets], nk[kMaxDenseTargets];
    int64_t sq[kMaxDenseTargets][3], so[kMaxDenseTargets][3];
};
static_assert(sizeof(MultiDenseArgs) <= 3072, "kernel arguments stay well inside the 4 KB kernarg space");

struct AttnF32Args {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* lse;
    int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t, sv_b, sv_h, sv_t, so_b, so_h, so_t;
    int32_t B, H;
    float scale_log2;
    const int32_t* kv_cnt;
    const int32_t* kv_idx;
    int32_t per_head;
    int32_t nqb, nkb;
    int32_t q_side;
    DevGeom g;
    int64_t nq, nk;
};

struct MaskArgs {
    DevGeom g;
    int32_t q_scale, n_sink, budget, keep_n, nkb;
    int32_t radius[kMaxScales];
    uint8_t* mask;
    int32_t* kv_cnt;
    int32_t* kv_idx;
};

struct ScoreArgs {
    const __bf16* q;
    const __bf16* k;
    float* scores;
    int64_t sq_b, sq_h, sq_t, sk_b, sk_h, sk_t;
    int32_t B, H;
    float scale_log2;
    int32_t d_side, nqb, nkb;
    DevGeom g;   // scales 0..D
};

constexpr int kMaxTargets = 8;   // target scales mapped by one select/map launch

struct SelMapArgs {
    DevGeom g;   // scales 0..largest target
    int32_t d_scale, n_sink, nqbD, nkbD, words;
    int32_t rule;     // 0: top-p (top_p), 1: Top-K fraction (k_keep tiles)
    int32_t k_keep;
    double top_p;
    const float* scores;
    int32_t* sel_cnt;   // written by target 0's waves when non-null
    int32_t* sel_idx;
    int32_t n_targets;
    int32_t groups_total;                   // sum over targets of ceil(nqbT / 4)
    int32_t t_scale[kMaxTargets], nqbT[kMaxTargets], nkbT[kMaxTargets];
    int32_t group_base[kMaxTargets + 1];    // prefix sums of ceil(nqbT / 4)
    int32_t* kv_cnt[kMaxTargets];
    int32_t* kv_idx[kMaxTargets];
};

struct OcacheArgs {
    const __bf16* o_full;      // decision scale, full attention output
    const __bf16* o_sparse;    // decision scale, sparse attention output
    __bf16* o_t;               // target scale, sparse output corrected in place
    int64_t sf_b, sf_h, sf_t, sp_b, sp_h, sp_t, so_b, so_h, so_t;
    int32_t B, H, head_dim, side_d, side_t;
};

struct JoinArgs {
    const int32_t* a_cnt;      // [sets or 1][rows]
    const int32_t* a_idx;      // [sets or 1][rows][nkb]
    const int32_t* b_cnt;
    const int32_t* b_idx;
    int32_t* out_cnt;          // [sets][rows]
    int32_t* out_idx;          // [sets][rows][nkb]
    int32_t sets, rows, nkb, words, join, a_per_set, b_per_set;
};

hipError_t launch_ocache_correct(const OcacheArgs& a, hipStream_t stream);
hipError_t launch_join_lists(const JoinArgs& a, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool dense, hipStream_t stream);
hipError_t launch_attn_multi_bf16(const MultiAttnArgs& m, int head_dim, hipStream_t stream);
hipError_t launch_dense_multi_bf16(const MultiDenseArgs& m, int head_dim, hipStream_t stream);
constexpr int kPairMaxNkbHost = 4096;   // key tiles the paired-tile kernel's LDS bitmaps cover
hipError_t launch_attn_pair_bf16(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_attn_fp32(const AttnF32Args& a, int head_dim, bool dense, hipStream_t stream);
hipError_t launch_csla_mask(const MaskArgs& a, int nqb, hipStream_t stream);
hipError_t launch_cs4a_score(const ScoreArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_cs4a_select_map(const SelMapArgs& a, int bh, hipStream_t stream);

}  // namespace vs

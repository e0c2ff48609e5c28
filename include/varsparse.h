/*
 * varsparse: block-sparse cross-scale attention for next-scale (VAR) image
 * generation on AMD Instinct MI355X (gfx950).
 *
 * The method is SparVAR's ("SparVAR: Exploring Sparsity in Visual
 * AutoRegressive Modeling for Training-Free Acceleration"; ai.info summary,
 * sections "Key Contributions", "Main Findings", "Methodology in Plain
 * English").  A query scale of the coarse-to-fine generation attends to the
 * concatenated key/value cache of every earlier scale plus itself.  The keys
 * a query tile may see are chosen per (query tile, key tile) pair:
 *   - CSLA: the first scales are attention sinks, visible to every query, and
 *     elsewhere a key is kept only inside a window around the query's
 *     projection onto the key's scale; the token mask is aggregated into tiles;
 *   - CS4A: attention is scored at a mid "decision" scale, the key tiles
 *     holding most of each query tile's attention mass are selected, and their
 *     indices are rescaled onto the later, larger scales.
 * Attention then runs over the kept tiles only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Scales are 0-based indices into geom->side[] (token-grid sides, strictly
 * ascending).  A query scale q attends to scales 0..q.  Tiles are square,
 * geom->tile tokens on a side, partial on the right/bottom edge of a grid
 * whose side is not a multiple of the tile.  Key tiles are numbered scale by
 * scale and in raster order within a scale; query tiles in raster order over
 * the query scale, whose side must be a multiple of the tile.
 *
 * Tensors are [B, H, N, head_dim] with the head dimension contiguous: the
 * caller passes element strides {batch, head, token}.  Q holds the N = side^2
 * tokens of the query scale in raster order; K and V hold the cache of scales
 * 0..q, concatenated, each in raster order (Nk = sum of side^2).  bf16 data
 * and its strides must be 16-byte aligned (strides multiples of 8 elements),
 * fp32 data 16-byte aligned (strides multiples of 4).
 *
 * Kept-tile lists: kv_cnt[r] is the number of kept key tiles of query tile r,
 * kv_idx[r * nkb + j] for j < kv_cnt[r] their ids in ascending order, the rest
 * of the row -1.  One list set is either shared by every (b, h) or given per
 * (b, h), laid out [B][H][nqb] and [B][H][nqb][nkb].
 *
 * Memory and errors: every pointer named "dev" is device memory owned by the
 * caller; the library allocates nothing and keeps no state except a
 * thread-local copy of the last HIP error.  Arguments are validated on the
 * host before anything is enqueued; a failed validation enqueues nothing and
 * returns VARSPARSE_EINVAL (malformed) or VARSPARSE_EUNSUPPORTED (valid but
 * outside what the kernels implement).  Work is enqueued on `stream` (a
 * hipStream_t; NULL = the default stream) and is asynchronous; a launch
 * failure returns VARSPARSE_EHIP.  No C++ exception crosses this interface.
 *
 * Empty inputs: B == 0 or H == 0 (varsparse_dense_attn_fwd: also nq == 0;
 * varsparse_join_lists: sets == 0) is valid.  Once the geometry and the
 * scalar arguments pass, such a call returns VARSPARSE_OK, enqueues nothing
 * and reads no data pointer, which may then be NULL.  Negative sizes are
 * EINVAL.
 */
#ifndef VARSPARSE_H
#define VARSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VARSPARSE_MAX_SCALES 32
#define VARSPARSE_MAX_ATTN_TARGETS 3   /* query scales of one varsparse_attn_fwd_multi call */
#define VARSPARSE_MAX_DENSE_TARGETS 16 /* query sets of one varsparse_dense_attn_fwd_multi call */

typedef struct varsparse_geom {
    int32_t n_scales;                      /* number of scales in side[]            */
    int32_t side[VARSPARSE_MAX_SCALES];    /* token-grid side of each scale, ascending */
    int32_t tile;                          /* tile side in tokens                   */
} varsparse_geom;

typedef enum varsparse_dtype {
    VARSPARSE_BF16 = 0,  /* bf16 inputs/outputs, fp32 accumulation (MFMA path) */
    VARSPARSE_FP32 = 1   /* fp32 inputs/outputs and arithmetic                 */
} varsparse_dtype;

enum {
    VARSPARSE_OK = 0,
    VARSPARSE_EINVAL = -1,
    VARSPARSE_EUNSUPPORTED = -2,
    VARSPARSE_EHIP = -3
};

/*
 * Tile and token counts of query scale q_scale (host only, no HIP call):
 * nqb query tiles, nkb key tiles of scales 0..q_scale, nq query tokens,
 * nk cached tokens.  Any output pointer may be NULL.
 */
int varsparse_geom_counts(const varsparse_geom* geom, int32_t q_scale,
                          int32_t* nqb, int32_t* nkb, int64_t* nq, int64_t* nk);

/*
 * CSLA window schedule (host only, no HIP call; SparVAR, ai.info summary,
 * "Main Findings", sink ablation item: window sizes [3, 5, 7] for the last 3
 * scales).  The last n_windows of n_scales query scales use windows[i] (odd,
 * >= 1, in tokens of each key scale) for query scale n_scales - n_windows + i:
 * radius[s] = (windows[i] - 1) / 2 for every key scale s = 0..q_scale.
 * radius: host array of q_scale + 1 entries, written.  EINVAL if q_scale is
 * not one of the last n_windows scales or a window is even or < 1.
 */
int varsparse_window_radius(int32_t n_scales, int32_t q_scale, const int32_t* windows, int32_t n_windows,
                            int32_t* radius);

/*
 * CSLA block mask of query scale q_scale, compacted to kept-tile lists
 * (SparVAR, ai.info summary, "Methodology in Plain English", second module;
 * "Main Findings", sink ablation).
 *
 * Radius mode (budget == -1): key tile K of scale s is kept for query tile Q
 * iff s < n_sink, or radius[s] >= 0 and some token pair of Q x K is within
 * the window: |y' - floor(y h/H)| <= radius[s] and |x' - floor(x h/H)| <=
 * radius[s], (y, x) a query token at side H, (y', x') a key token at side h.
 * radius: host array of q_scale + 1 entries, in tokens of each key scale;
 * a negative entry drops that scale (sinks excepted).
 *
 * Budget mode (budget > 0, radius ignored and may be NULL): per query tile
 * keep the first max(budget, sink tiles + 1) key tiles (at most nkb) ranked by
 * (not sink, admission radius, -scale, id), the admission radius being the
 * smallest window radius that keeps the pair.  Supports nkb <= 4096.
 *
 * Outputs (dev): mask u8 [nqb * nkb] (1 = kept; may be NULL), kv_cnt int32
 * [nqb], kv_idx int32 [nqb * nkb] (ascending, -1 padded).  0 <= n_sink <= q_scale.
 * Bit-exact integer work; the lists are shared by every (batch, head).
 */
int varsparse_build_mask(const varsparse_geom* geom, int32_t q_scale, int32_t n_sink,
                         const int32_t* radius, int32_t budget,
                         uint8_t* mask, int32_t* kv_cnt, int32_t* kv_idx, void* stream);

/*
 * CS4A mask prediction (SparVAR, ai.info summary, "Methodology in Plain
 * English", first module; "Main Findings", decision scale) for target scale
 * t_scale from decision scale d_scale (d_scale <= t_scale, both sides
 * multiples of the tile, 0 <= n_sink <= d_scale, 0 < top_p <= 1).
 *
 * Scoring (run when q_d != NULL): P = softmax(Q_D K^T * softmax_scale) over
 * the keys of scales 0..d_scale, per (b, h); scores[b][h][Q][K] =
 * (1/|Q|) * sum of P over the pairs of query tile Q and key tile K (each row
 * sums to 1).  q_d: dev [B, H, side_D^2, head_dim] with strides q_strides;
 * k: dev, the key cache (only its first sum_{s<=D} side^2 tokens are read),
 * strides k_strides.  bf16 only, head_dim in {64, 128}, tile == 8.
 * With q_d == NULL, scores are an input (a previous call's output) and k,
 * q_strides, k_strides, softmax_scale are ignored.
 * scores: dev float32 [B * H * nqb_D * nkb_D], nkb_D <= 240.
 *
 * Selection: per (b, h, decision query tile) the scores are quantised to
 * m = floor(score * 2^24), ordered by (m descending, id ascending), and the
 * shortest prefix whose sum reaches ceil(top_p * sum m) (IEEE double) is kept.
 * sel_cnt int32 [B*H*nqb_D] and sel_idx int32 [B*H*nqb_D*nkb_D] (ascending,
 * -1 padded) receive it when both are non-NULL.
 *
 * Mapping: target query tile (i, j) takes the selection of decision tile
 * (floor(i nb_D/nb_T), floor(j nb_D/nb_T)); selected tiles of scales below D
 * are kept; a selected tile of scale D becomes, on every scale s with
 * D <= s <= t_scale, the tiles covering token rows
 * [floor(a t h_s/h_D), ceil(e h_s/h_D) - 1] (e the tile's end row) and the
 * same columns; the sink tiles (scales < n_sink) are added.
 * kv_cnt int32 [B*H*nqb_T], kv_idx int32 [B*H*nqb_T*nkb_T] (per-(b, h) lists).
 */
int varsparse_map_indices(const varsparse_geom* geom, int32_t d_scale, int32_t t_scale,
                          int32_t n_sink, float top_p, varsparse_dtype dtype,
                          int32_t B, int32_t H, int32_t head_dim,
                          const void* q_d, const int64_t q_strides[3],
                          const void* k, const int64_t k_strides[3], float softmax_scale,
                          float* scores, int32_t* sel_cnt, int32_t* sel_idx,
                          int32_t* kv_cnt, int32_t* kv_idx, void* stream);

/*
 * CS4A with the Top-K-fraction selection rule (SparVAR, ai.info summary,
 * "Main Findings", decision-scale item: a Top-K ratio of about 0.2 is the
 * stable setting; "Methodology in Plain English", first module: a Top-K
 * operation picks the key blocks).  Identical to varsparse_map_indices except
 * for the selection: per decision query tile the first
 * k = min(max(ceil(top_k_frac * nkb_D), 1), nkb_D) key tiles (the product in
 * IEEE single precision) of the order (m descending, id ascending) are kept.
 * 0 < top_k_frac <= 1.
 */
int varsparse_map_indices_topk(const varsparse_geom* geom, int32_t d_scale, int32_t t_scale,
                               int32_t n_sink, float top_k_frac, varsparse_dtype dtype,
                               int32_t B, int32_t H, int32_t head_dim,
                               const void* q_d, const int64_t q_strides[3],
                               const void* k, const int64_t k_strides[3], float softmax_scale,
                               float* scores, int32_t* sel_cnt, int32_t* sel_idx,
                               int32_t* kv_cnt, int32_t* kv_idx, void* stream);

/*
 * Block-sparse attention of query scale q_scale over its cache (SparVAR,
 * ai.info summary, "Key Contributions" item 3 and "Main Findings", the
 * block-wise sparse kernel).  For every query of tile Q:
 *     O = softmax(q K_kept^T * softmax_scale) V_kept,
 *     lse = log(sum over kept keys of exp(q k * softmax_scale)),
 * K_kept / V_kept the tokens of the kept key tiles of Q.  A query tile with no
 * kept tile gets O = 0 and lse = -inf.
 *
 * q, o: dev [B, H, side_q^2, head_dim]; k, v: dev [B, H, Nk, head_dim];
 * strides: 12 element strides {q_b, q_h, q_t, k_b, k_h, k_t, v_b, v_h, v_t,
 * o_b, o_h, o_t}.  lse: dev float32 [B, H, side_q^2] contiguous, or NULL.
 * kv_cnt / kv_idx: dev lists as above; lists_per_head = 0 for one set shared
 * by every (b, h), 1 for per-(b, h) lists.  kv_idx entries must be valid,
 * ascending key-tile ids.
 * bf16: head_dim in {64, 128}, tile == 8 (64-query tiles).
 * fp32: head_dim in {64, 128}, tile * tile <= 64.
 */
int varsparse_attn_fwd(const varsparse_geom* geom, int32_t q_scale, varsparse_dtype dtype,
                       int32_t B, int32_t H, int32_t head_dim,
                       const void* q, const void* k, const void* v, void* o, float* lse,
                       const int64_t strides[12], float softmax_scale,
                       const int32_t* kv_cnt, const int32_t* kv_idx, int32_t lists_per_head,
                       void* stream);

/* Selection rule of varsparse_map_indices_multi. */
enum {
    VARSPARSE_SELECT_TOP_P = 0,   /* param = p, as varsparse_map_indices       */
    VARSPARSE_SELECT_TOP_K = 1    /* param = fraction, as varsparse_map_indices_topk */
};

/*
 * CS4A scoring, selection and index mapping onto several target scales in one
 * launch (SparVAR, ai.info summary, "Methodology in Plain English", first
 * module: the indices selected at the decision scale are mapped to the later
 * scales; all of them depend only on the decision scale, so they are built
 * together right after it).  For each i < n_targets the lists of target
 * scale t_scales[i] are exactly those varsparse_map_indices (rule 0) or
 * varsparse_map_indices_topk (rule 1) writes for that target: kv_cnt[i] dev
 * int32 [B*H*nqb_T], kv_idx[i] dev int32 [B*H*nqb_T*nkb_T].  kv_cnt, kv_idx,
 * t_scales: host arrays of n_targets entries (1 <= n_targets <= 8), each
 * target d_scale <= t < n_scales.  Scores as in varsparse_map_indices
 * (computed when q_d is non-NULL, else read).  No selection output.
 */
int varsparse_map_indices_multi(const varsparse_geom* geom, int32_t d_scale, int32_t n_targets,
                                const int32_t* t_scales, int32_t n_sink, int32_t rule, float param,
                                varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim,
                                const void* q_d, const int64_t q_strides[3], const void* k,
                                const int64_t k_strides[3], float softmax_scale, float* scores,
                                int32_t* const* kv_cnt, int32_t* const* kv_idx, void* stream);

/*
 * Block-sparse attention with 128-query workgroups (SparVAR, ai.info
 * summary, "Main Findings": the block-wise kernel measured with blocks of
 * 128 and of 64 tokens).  Same operation, arguments, layouts and results
 * (up to rounding order) as varsparse_attn_fwd with dtype VARSPARSE_BF16:
 * query tiles 2p and 2p + 1 share one workgroup that walks the union of
 * their kept-tile lists, loads every key chunk once for both and attends
 * each tile to its own list only.  tile == 8, head_dim in {64, 128}; at
 * most 4096 key tiles (VARSPARSE_EUNSUPPORTED above).  On MI355X this form
 * measures 0.8-0.9x the speed of varsparse_attn_fwd on the last-scale
 * workload (a chunk kept by one tile of the pair idles the other tile's
 * waves at its barrier), so every other path uses the 64-query kernel; it
 * is kept to compare the pages' two block sizes, not as their setting.
 */
int varsparse_attn_fwd_pair(const varsparse_geom* geom, int32_t q_scale, int32_t B, int32_t H, int32_t head_dim,
                            const void* q, const void* k, const void* v, void* o, float* lse,
                            const int64_t strides[12], float softmax_scale, const int32_t* kv_cnt,
                            const int32_t* kv_idx, int32_t lists_per_head, void* stream);

/*
 * Token-exact CSLA attention (SparVAR, ai.info summary, "Methodology in Plain
 * English", second module: the token-level sink + window mask; "Key
 * Contributions" item 3: the naive token-wise sparse attention baseline).
 * For every query of tile Q: softmax over the keys the token rule keeps
 * (scale s < n_sink, or radius[s] >= 0 and |y' - floor(y h/H)| <= radius[s]
 * and |x' - floor(x h/H)| <= radius[s]), times V, and lse as in
 * varsparse_attn_fwd; a query keeping no key gets O = 0 and lse = -inf.
 * With lists (kv_cnt, kv_idx as in varsparse_attn_fwd, e.g. the CSLA block
 * mask of the same n_sink and radius) only the listed tiles are walked and the
 * token rule is applied inside them; the result is the same as long as every
 * kept token pair lies in a listed tile.  With kv_cnt = kv_idx = NULL every key
 * tile is walked: the token-masked dense baseline.
 * radius: host array of q_scale + 1 entries.  bf16, head_dim in {64, 128},
 * tile == 8, query side <= 4096 (VARSPARSE_EUNSUPPORTED above: the
 * projections are exact integer quotients below 2^24); layouts and strides
 * as varsparse_attn_fwd.
 */
int varsparse_attn_fwd_token(const varsparse_geom* geom, int32_t q_scale, int32_t n_sink,
                             const int32_t* radius, int32_t B, int32_t H, int32_t head_dim,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int64_t strides[12], float softmax_scale,
                             const int32_t* kv_cnt, const int32_t* kv_idx, int32_t lists_per_head,
                             void* stream);

/*
 * Dense attention written with the same tile engine, the comparator the
 * pages measure the sparse kernel against ("Main Findings": the block-wise
 * kernel vs dense FlashAttention on the last scale).  Every query attends to
 * all nk keys.  Layouts and lse as for varsparse_attn_fwd; nq >= 0, nk >= 1.
 * bf16 or fp32, head_dim in {64, 128}.  A bf16 launch of at most 512 blocks of
 * 64 queries (B * H * ceil(nq / 64)) over at least 384 keys splits each block's
 * keys over 2 or 4 wave groups and merges their partial softmaxes: the same
 * result up to rounding order.
 */
int varsparse_dense_attn_fwd(varsparse_dtype dtype, int32_t B, int32_t H, int32_t head_dim,
                             int64_t nq, int64_t nk,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int64_t strides[12], float softmax_scale, void* stream);

/*
 * O_cache correction (SparVAR, ai.info summary, "Methodology in Plain
 * English", first module: the decision scale's leftover output is cached and
 * upsampled to correct the later sparse outputs; "Main Findings", the item on
 * the two modules' increments).  For every (b, h), target token (y, x) and
 * head dim c:
 *     o_t[y, x, c] += o_full_d[y', x', c] - o_sparse_d[y', x', c],
 *     y' = floor(y side_d / side_t), x' = floor(x side_d / side_t),
 * with o_full_d / o_sparse_d the decision scale's full and block-sparse
 * attention outputs and o_t the target scale's block-sparse output, updated
 * in place (fp32 arithmetic, one rounding to bf16).
 * All three: dev bf16 [B, H, side^2, head_dim], head dim contiguous, 16-byte
 * aligned; strides: 9 element strides {full_b, full_h, full_t, sparse_b,
 * sparse_h, sparse_t, t_b, t_h, t_t}, multiples of 8.  1 <= side_d <= side_t,
 * head_dim a multiple of 8; o_t must not overlap the two decision outputs.
 */
int varsparse_ocache_correct(int32_t B, int32_t H, int32_t head_dim, int32_t side_d, int32_t side_t,
                             const void* o_full_d, const void* o_sparse_d, void* o_t,
                             const int64_t strides[9], void* stream);

/*
 * Block-sparse attention of a later scale with its O_cache correction, in one
 * pass (SparVAR, ai.info summary, "Methodology in Plain English", first
 * module: the later sparse outputs are corrected with the decision scale's
 * cached residual).  For every query (y, x) of query scale q_scale and head
 * dim c:
 *     o[y, x, c] = A[y, x, c] + o_full_d[y', x', c] - o_sparse_d[y', x', c],
 *     y' = floor(y side_d / side_q), x' = floor(x side_d / side_q),
 * with A the attention varsparse_attn_fwd computes (same arguments, lists
 * and lse) and side_d the side of decision scale d_scale <= q_scale: the
 * result of varsparse_attn_fwd followed by varsparse_ocache_correct, with the
 * sum taken in fp32 and rounded to bf16 once (not after the attention too).
 * bf16 only, head_dim in {64, 128}, tile == 8.  o_full_d / o_sparse_d: dev
 * bf16 [B, H, side_d^2, head_dim], 16-byte aligned, not overlapping o;
 * d_strides: 6 element strides {full_b, full_h, full_t, sparse_b, sparse_h,
 * sparse_t}, multiples of 8.
 */
int varsparse_attn_fwd_ocache(const varsparse_geom* geom, int32_t q_scale, int32_t d_scale, int32_t B, int32_t H,
                              int32_t head_dim, const void* q, const void* k, const void* v, void* o, float* lse,
                              const int64_t strides[12], float softmax_scale, const int32_t* kv_cnt,
                              const int32_t* kv_idx, int32_t lists_per_head, const void* o_full_d,
                              const void* o_sparse_d, const int64_t d_strides[6], void* stream);

/*
 * Block-sparse attention of several query scales over one cache in one
 * launch (SparVAR, ai.info summary, "Methodology in Plain English", first
 * module: the lists mapped from one decision scale serve all the later
 * scales, whose attentions are independent of one another).  For each
 * i < n_targets, target i gets exactly (bit for bit) what varsparse_attn_fwd
 * with dtype VARSPARSE_BF16 writes for query scale q_scales[i], with q[i],
 * o[i], lse[i] (lse NULL, or lse[i] NULL: none), strides + 12 i, kv_cnt[i] and
 * kv_idx[i]; when o_full_d is non-NULL, what varsparse_attn_fwd_ocache writes
 * with the decision scale d_scale <= every q_scales[i] and its outputs
 * o_full_d / o_sparse_d (d_strides as there; both NULL: no correction).
 * Host arrays: q_scales, q, o, lse, kv_cnt, kv_idx (n_targets entries each),
 * strides (12 * n_targets entries; the K and V entries 3..8 equal for every
 * target: one cache).  1 <= n_targets <= VARSPARSE_MAX_ATTN_TARGETS; every
 * target scale a multiple of the tile side, tile == 8, bf16, head_dim in
 * {64, 128}; lists_per_head applies to every target.  Outputs of different
 * targets must not overlap.  EINVAL / EUNSUPPORTED as for varsparse_attn_fwd,
 * nothing enqueued.
 */
int varsparse_attn_fwd_multi(const varsparse_geom* geom, int32_t n_targets, const int32_t* q_scales, int32_t B,
                             int32_t H, int32_t head_dim, const void* const* q, const void* k, const void* v,
                             void* const* o, float* const* lse, const int64_t* strides, float softmax_scale,
                             const int32_t* const* kv_cnt, const int32_t* const* kv_idx, int32_t lists_per_head,
                             int32_t d_scale, const void* o_full_d, const void* o_sparse_d,
                             const int64_t d_strides[6], void* stream);

/*
 * Dense attention of several query sets over prefixes of one cache in one
 * launch (SparVAR, ai.info summary, "Methodology in Plain English": the early
 * scales are attended densely; each scale's queries see the cache of every
 * scale up to their own).  Target i gets the dense attention that
 * varsparse_dense_attn_fwd with dtype VARSPARSE_BF16 computes for nq[i]
 * queries q[i] over the first nk[i] keys of k and v, into o[i] and lse[i]
 * (lse NULL, or lse[i] NULL: none), with strides + 12 i (the K and V entries
 * 3..8 equal for every target): every 64-query block walks its keys in one
 * pass, so the result is bit-identical to that call wherever the call does
 * the same (it splits a block's keys over wave pairs, summing in another
 * order, when it has at most 512 blocks of 12 or more 32-key chunks).  Host arrays of n_targets entries: nq, nk, q,
 * o, lse, and 12 * n_targets strides.  1 <= n_targets <=
 * VARSPARSE_MAX_DENSE_TARGETS, nq[i] >= 0 (0: nothing for that target),
 * nk[i] >= 1; bf16, head_dim in {64, 128}.  Outputs of different targets
 * must not overlap.  EINVAL / EUNSUPPORTED as for varsparse_dense_attn_fwd,
 * nothing enqueued.
 */
int varsparse_dense_attn_fwd_multi(int32_t n_targets, int32_t B, int32_t H, int32_t head_dim, const int64_t* nq,
                                   const int64_t* nk, const void* const* q, const void* k, const void* v,
                                   void* const* o, float* const* lse, const int64_t* strides, float softmax_scale,
                                   void* stream);

/* Static description of a status code. */
/* How varsparse_join_lists combines two kept-tile sets. */
enum {
    VARSPARSE_JOIN_UNION = 0,
    VARSPARSE_JOIN_INTERSECTION = 1
};

/*
 * Join of two kept-tile lists per query tile (SparVAR, ai.info summary,
 * "Main Findings": CS4A, its O_cache correction and CSLA are used together,
 * CSLA with windows 3/5/7 on the last three scales; "Methodology in Plain
 * English": CSLA builds its mask without the decision scale).  Used to join a
 * query scale's CS4A-mapped lists (per (b, h)) with its CSLA lists (shared by
 * every head).  out row = a row ∪ b row (join 0) or a row ∩ b row (join 1),
 * ascending, -1 padded to nkb entries; integer only, bit-exact.
 * Lists (dev int32): cnt [sets][rows], idx [sets][rows][nkb], ascending ids
 * without repeats; a_per_set / b_per_set = 0 means one list set [rows] shared
 * by every set.  Entries outside [0, nkb) are ignored and counts are clamped
 * to [0, nkb].  out_cnt [sets][rows], out_idx [sets][rows][nkb] must not
 * overlap the inputs.  1 <= nkb <= 65536, sets * rows < 2^31; EINVAL
 * otherwise, nothing enqueued.
 */
int varsparse_join_lists(int32_t sets, int32_t rows, int32_t nkb, int32_t join,
                         const int32_t* a_cnt, const int32_t* a_idx, int32_t a_per_set,
                         const int32_t* b_cnt, const int32_t* b_idx, int32_t b_per_set,
                         int32_t* out_cnt, int32_t* out_idx, void* stream);

const char* varsparse_strerror(int code);

/* The hipError_t of the calling thread's last VARSPARSE_EHIP (0 if none). */
int varsparse_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VARSPARSE_H */

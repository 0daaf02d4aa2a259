/*
 * cacheblend.h -- C ABI of the MI355X (gfx950) CacheBlend KV-fusion library.
 *
 * One layer of the blend joins separately prefilled chunk caches of a request:
 *   1. cached keys are moved to their new positions by re-rotation,
 *   2. each candidate token is scored by the squared deviation of its V row,
 *   3. the top-k tokens per request are selected,
 *   4. their recomputed K/V rows replace the cached rows,
 *   5. the selected query rows run causal GQA attention over the fused cache.
 *
 * Pages cited:
 *   [Derivations] the page "数学推导" (math derivations) of the CacheBlend
 *                 documentation, inference.lei6393.com/cacheblend/appendix/
 *                 c-math-derivations/
 *   [KV-blog]     the blog page "rag的kvcache问题" (zxj-2023.github.io)
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the argument says [host].
 *   - Tensors are dense, row-major and token-major: [token][head][dim].
 *     Element type is cb_geom.dtype (fp32 or bf16); every base pointer of a
 *     tensor must be 16-byte aligned.  Index arrays are int32.
 *   - "Packed" rows: the tokens of all requests of a ragged batch are
 *     concatenated; request r owns rows [tok_off[r], tok_off[r+1]).  Positions
 *     inside a request start at 0.
 *   - Candidate rows: request r's candidates are cand_idx[cand_off[r] ..
 *     cand_off[r+1]), packed row numbers in ascending order; the recomputed
 *     tensors (k_new_c, v_new_c, q_c) hold one row per candidate in that order.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates, frees or synchronizes, and keeps no mutable global
 *     state, except the static device scratch of cb_blend_layer_noalloc.
 *   - Ordering: every call enqueues its kernels on `stream` (a hipStream_t;
 *     NULL = the default stream) and returns without waiting.  Calls are
 *     thread-safe.
 *   - Errors: argument errors are detected on the host before any HIP call and
 *     return CB_ERR_INVALID_ARG or CB_ERR_UNSUPPORTED with nothing enqueued.
 *     A failed launch returns CB_ERR_HIP.  cb_last_error() gives the detail
 *     text of the calling thread's last failure.  Device-side preconditions
 *     that the host cannot see (index values in range, ascending order) are
 *     the caller's responsibility.
 */
#ifndef CACHEBLEND_H
#define CACHEBLEND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cb_status {
  CB_OK = 0,
  CB_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or offsets */
  CB_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  CB_ERR_HIP = 3          /* the HIP runtime reported an error */
} cb_status;

typedef enum cb_dtype { CB_DTYPE_F32 = 0, CB_DTYPE_BF16 = 1 } cb_dtype;

/* Pairing of the coordinates that one RoPE 2x2 block rotates. */
typedef enum cb_rope_style {
  CB_ROPE_HALF = 0,        /* pairs (j, j + D/2), j < D/2 */
  CB_ROPE_INTERLEAVED = 1  /* pairs (2j, 2j + 1) */
} cb_rope_style;

/* What the deviation of a candidate token measures.  V alone is the score of
 * [Derivations, "近似解"]; [KV-blog, "核心发现： KV 偏差"] speaks of the
 * distance between the token's whole KV vectors (cached vs recomputed).  Keys
 * are compared at the new position: the cached key after re-rotation. */
typedef enum cb_dev_source {
  CB_DEV_V = 0,  /* ||V_new - V_old||^2 */
  CB_DEV_K = 1,  /* ||K_new - K_cached||^2 */
  CB_DEV_KV = 2  /* the K and V rows read as one vector: the sum of both */
} cb_dev_source;

/* Head geometry.  n_q_heads % n_kv_heads == 0; query head h reads KV head
 * h / (n_q_heads / n_kv_heads).  head_dim in {16, 32, 64, 128}. */
typedef struct cb_geom {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* cb_dtype */
} cb_geom;

/* A ragged batch of n_req independent requests.  The three offset arrays have
 * n_req + 1 entries, start at 0 and never decrease.  The device copies feed
 * the kernels; the [host] mirrors (same values) serve validation and grid
 * sizing, so no call ever reads device memory back. */
typedef struct cb_ragged {
  int32_t n_req;
  const int32_t *tok_off;    /* packed token rows of each request */
  const int32_t *cand_off;   /* candidate slice of each request */
  const int32_t *sel_off;    /* selected slice: k_r = sel_off[r+1] - sel_off[r] */
  const int32_t *h_tok_off;  /* [host] */
  const int32_t *h_cand_off; /* [host] */
  const int32_t *h_sel_off;  /* [host] */
} cb_ragged;

/*
 * cb_rerotate -- move cached keys to their new positions.
 * [Derivations, "CacheBlend 中的应用"]: a key cached at p_old is taken to
 * p_new by the rotation R_{p_new - p_old}; R is the block-diagonal matrix of
 * 2x2 rotations of [Derivations, "RoPE 位置编码的相对位置不变性证明"], pair j
 * turning by delta * theta^(-2j/D) (the RoFormer schedule).  V is not rotated.
 *
 *   k_in, k_out : [n_layers][n_tok][n_kv_heads][head_dim], dtype.  k_out may
 *                 equal k_in (in place); any other overlap is invalid.  In place,
 *                 rows whose delta is 0 are not touched; out of place they are
 *                 copied unchanged.
 *   delta       : [n_tok] int32, p_new - p_old of each packed row (shared by
 *                 all layers).
 *   rope_theta  : frequency base (> 0, finite).
 * Angles are reduced in double precision, the rotation is applied in fp32 and
 * stored with round-to-nearest-even.
 */
cb_status cb_rerotate(const cb_geom *geom, void *k_out, const void *k_in,
                      const int32_t *delta, int64_t n_tok, int32_t n_layers,
                      double rope_theta, int32_t rope_style, void *stream);

/*
 * cb_deviation_topk -- score candidates and select the high-deviation tokens.
 * [Derivations, "近似解"]: S = TopK_i ||V_new[i] - V_old[i]||_2^2, summed
 * over every KV head and dimension of the token; [KV-blog, "渐进式过滤机制"]:
 * the candidate pool is all tokens at layer 1 and the survivors afterwards.
 *
 *   v_new_c  : [M][n_kv_heads][head_dim]  recomputed V of the candidates
 *   v_old    : [T][n_kv_heads][head_dim]  cached V (T = h_tok_off[n_req])
 *   cand_idx : [M] candidate packed rows (M = h_cand_off[n_req])
 *   dev      : [M] fp32 out, the deviation of each candidate (fp32 accumulation)
 *   sel_local, sel_global : [K] int32 out (K = h_sel_off[n_req]).  For request
 *              r, the k_r candidates with the largest deviation (NaN above
 *              +inf; ties to the lower packed row), in ascending order:
 *              sel_local = index into the candidate arrays (0 .. M-1),
 *              sel_global = cand_idx[sel_local].
 * Requires k_r <= M_r <= N_r for every request.
 */
cb_status cb_deviation_topk(const cb_geom *geom, const cb_ragged *rg,
                            const void *v_new_c, const void *v_old,
                            const int32_t *cand_idx, float *dev,
                            int32_t *sel_local, int32_t *sel_global,
                            void *stream);

/*
 * cb_kv_deviation_topk -- cb_deviation_topk with the deviation taken on the
 * part of the token's KV that `source` (cb_dev_source) names; same selection
 * and output rules.
 *
 *   k_new_c  : [M][n_kv_heads][head_dim]  recomputed K of the candidates
 *   k_cached : [T][n_kv_heads][head_dim]  cached K, already re-rotated to the
 *              new positions (cb_rerotate)
 *   v_new_c, v_old, cand_idx, dev, sel_local, sel_global : as cb_deviation_topk.
 * The K pointers may be NULL for CB_DEV_V, the V pointers for CB_DEV_K.  An
 * unknown source returns CB_ERR_INVALID_ARG.
 */
cb_status cb_kv_deviation_topk(const cb_geom *geom, const cb_ragged *rg, int32_t source,
                               const void *k_new_c, const void *k_cached,
                               const void *v_new_c, const void *v_old,
                               const int32_t *cand_idx, float *dev,
                               int32_t *sel_local, int32_t *sel_global, void *stream);

/*
 * cb_topk -- the selection half of cb_deviation_topk on given fp32 scores:
 * same ordering, tie and output rules.  dev: [M] fp32.
 */
cb_status cb_topk(const cb_ragged *rg, const float *dev, const int32_t *cand_idx,
                  int32_t *sel_local, int32_t *sel_global, void *stream);

/*
 * cb_fuse_scatter -- splice the recomputed rows into the cache, in place.
 * [Derivations, "形式化"]: K_fused[i] = K_new[i] for i in S, else the cached
 * row; V likewise.  [KV-blog, "渐进式过滤机制"]: the recomputed rows are
 * joined with the reused cache before attention.
 *
 *   k_fused, v_fused : [T][n_kv_heads][head_dim], in/out (hold K_rot / V_old)
 *   k_new_c, v_new_c : [M][n_kv_heads][head_dim]
 *   sel_local, sel_global : [k_total]; row sel_local[s] of the new tensors is
 *                    copied bit for bit to row sel_global[s] of the fused ones.
 */
cb_status cb_fuse_scatter(const cb_geom *geom, void *k_fused, void *v_fused,
                          const void *k_new_c, const void *v_new_c,
                          const int32_t *sel_local, const int32_t *sel_global,
                          int64_t k_total, void *stream);

/*
 * cb_rerotate_fuse -- cb_rerotate (one layer, in place) followed by
 * cb_fuse_scatter, in one pass after the selection: the rows of S take the
 * recomputed K and V rows, and only the other rows' K is re-rotated.
 * [Derivations, "形式化"]: a token outside S keeps its cached row and a token
 * in S takes its recomputed row, so the rotation of [Derivations,
 * "CacheBlend 中的应用"] is wasted on the rows of S.  For row t:
 *   k[t] = t in S ? k_new_c[sel_local[s]] : R_{delta[t]} k[t]  (s: sel_global[s] = t)
 *   v[t] = t in S ? v_new_c[sel_local[s]] : v[t]
 * The result is bit for bit that of cb_rerotate then cb_fuse_scatter.
 *   k, v           : [n_tok][n_kv_heads][head_dim], in/out
 *   k_new_c, v_new_c : [M][n_kv_heads][head_dim]
 *   delta          : [n_tok] p_new - p_old (not NULL when n_tok > 0)
 *   sel_local, sel_global : [k_total]; sel_global strictly ascending over the
 *                    whole packed batch (as cb_deviation_topk writes it), not
 *                    checked on the host.
 * Errors: those of cb_rerotate and cb_fuse_scatter; INVALID_ARG if
 * k_total > n_tok.
 */
cb_status cb_rerotate_fuse(const cb_geom *geom, void *k, void *v, const void *k_new_c,
                           const void *v_new_c, const int32_t *delta,
                           const int32_t *sel_local, const int32_t *sel_global,
                           int64_t k_total, int64_t n_tok, double rope_theta,
                           int32_t rope_style, void *stream);

/*
 * cb_partial_attn -- causal GQA attention of the selected rows only.
 * [Derivations, "形式化"]: Attention(Q, K_fused, V_fused); [KV-blog, "阶段二：
 * 注意力分数计算阶段"]: every query row is computed independently;
 * [KV-blog, "transformer训练与推理并行计算的差异"]: causal mask.
 *
 * For selected row s of request r (packed row p = sel_global[s]) and query
 * head h, with g = h / (n_q_heads / n_kv_heads):
 *   out[s][h] = sum_{u = tok_off[r]}^{p} softmax_u(<q, K_fused[u][g]> * scale)
 *               * V_fused[u][g],   q = q_c[sel_local[s]][h].
 *   out    : [K][n_q_heads][head_dim] dtype, K = h_sel_off[n_req]
 *   q_c    : [M][n_q_heads][head_dim], already rotated at the new positions
 *   workspace, workspace_bytes : optional device scratch owned by the caller
 *            (NULL/0 allowed).  When the query tiles are too few to fill the
 *            GPU, long rows are split over key ranges whose partials
 *            live here, with one arrival counter per query tile and KV head
 *            (the last chunk to arrive merges them and sets its counter
 *            back to zero; the call clears the counters first, so the
 *            contents need no initialisation);
 *            cb_partial_attn_workspace_size() gives the size that enables
 *            the split.  A smaller workspace only disables the split.
 *            Calls that share a workspace must be ordered on one stream.
 * bf16 uses MFMA products with fp32 accumulation and an fp32 online softmax.
 */
cb_status cb_partial_attn(const cb_geom *geom, const cb_ragged *rg, void *out,
                          const void *q_c, const int32_t *sel_local,
                          const int32_t *sel_global, const void *k_fused,
                          const void *v_fused, float softmax_scale,
                          void *workspace, size_t workspace_bytes,
                          void *stream);

/* Workspace (bytes) with which cb_partial_attn can split long rows for this
 * geometry and batch; 0 when no split is used.  Reads host mirrors only. */
cb_status cb_partial_attn_workspace_size(const cb_geom *geom,
                                         const cb_ragged *rg, size_t *bytes);

/* How cb_partial_attn decomposes the work for a geometry and batch. */
typedef struct cb_attn_plan {
  int32_t mfma;           /* 1: bf16 MFMA query tiles; 0: plain kernel (one
                             wave per selected row and query head) */
  int32_t key_split;      /* MFMA: wave groups that split the keys of every
                             tile (1: 256 query vectors, 64-key tiles;
                             2: 128 query vectors, 128-key tiles) */
  int32_t rows_per_tile;  /* MFMA: selected rows per query tile */
  int32_t key_chunk;      /* MFMA: keys per chunk when long rows are split over
                             keys (their partials go to the workspace); 0: no split */
  int64_t tiles;          /* MFMA: query tiles over all requests */
  int64_t workgroups;     /* workgroups of the attention launch (launched
                             longest piece first when the plan is split and
                             has at most 960 units; the order never changes
                             the result) */
  size_t workspace_bytes; /* workspace the plan uses (<= the size passed in) */
  int32_t stream_spans;   /* MFMA, key split 1: > 0 = balanced decomposition --
                             the 64-key tiles of all query tiles of a KV head,
                             laid end to end, are cut into this many equal
                             spans, one workgroup each; a query tile cut by a
                             span's end is computed in pieces whose partials
                             merge as key chunks do.  0: (query tile, key
                             chunk) workgroups.  cb_partial_attn never chooses
                             it (slower on the shapes measured); a pinned plan
                             may. */
} cb_attn_plan;

/* The plan cb_partial_attn follows with `workspace_bytes` of workspace
 * (SIZE_MAX: as with cb_partial_attn_workspace_size()).  The choice is a
 * host-side cost model of the launch; it reads host mirrors only and
 * enqueues nothing.  Errors: INVALID_ARG for a NULL plan or invalid
 * geometry / offsets (the plan is zeroed first). */
cb_status cb_partial_attn_plan(const cb_geom *geom, const cb_ragged *rg,
                               size_t workspace_bytes, cb_attn_plan *plan);

/* Completes a pinned plan: reads mfma, key_split and key_chunk, checks them
 * as cb_partial_attn_with_plan does (same errors; *plan unchanged on error)
 * and fills the other fields, workspace_bytes included.  Host only. */
cb_status cb_partial_attn_describe_plan(const cb_geom *geom, const cb_ragged *rg,
                                        cb_attn_plan *plan);

/*
 * cb_partial_attn_with_plan -- cb_partial_attn with the decomposition pinned
 * by the caller instead of chosen by the cost model (tuning, reproducible
 * launch shapes).  Same operation, arguments and result as cb_partial_attn.
 * Of *plan only four fields are read:
 *   mfma      : 0 = plain kernel (any geometry), 1 = MFMA query tiles;
 *   key_split : 1 or 2 (MFMA); UNSUPPORTED if the group size does not
 *               divide the 256 / key_split query vectors of a tile;
 *   key_chunk : 0 = no split over keys, else a positive multiple of
 *               64 * key_split that splits no request with selected rows
 *               into more than 8 chunks (INVALID_ARG otherwise);
 *   stream_spans : 0, or 1 .. 65536 spans of the balanced decomposition
 *               (key_split 1 and key_chunk 0, else INVALID_ARG; at most
 *               1024 requests and 2048 query tiles, else UNSUPPORTED).
 * A split needs the workspace that cb_partial_attn_describe_plan() reports
 * for the same fields (INVALID_ARG if workspace_bytes is smaller).
 *
 * flags : 0 or CB_ATTN_COUNTERS_ZERO (other bits: INVALID_ARG).  Without it
 *   a split plan first clears its arrival counters with a small launch of
 *   its own, as cb_partial_attn does.  Every call leaves its plan's counters
 *   at zero, so a caller that fills the workspace with zeros once and then
 *   calls with one plan on it may pass the flag and save that launch.  The
 *   partials of a different split plan on the same workspace can overwrite
 *   this plan's counters: after such a call fill with zeros again, or omit
 *   the flag.  Counters that are not zero under the flag give wrong output
 *   rows (a tile merged early or never); nothing waits on them, so nothing
 *   hangs.  Unsplit plans use no counters and ignore the flag.
 */
#define CB_ATTN_COUNTERS_ZERO 1u
cb_status cb_partial_attn_with_plan(const cb_geom *geom, const cb_ragged *rg,
                                    const cb_attn_plan *plan, void *out,
                                    const void *q_c, const int32_t *sel_local,
                                    const int32_t *sel_global, const void *k_fused,
                                    const void *v_fused, float softmax_scale,
                                    void *workspace, size_t workspace_bytes,
                                    uint32_t flags, void *stream);

/* Order of the steps in cb_blend_layer.
 *   CB_ORDER_ROTATE_FIRST : re-rotate, score, select, fuse; the re-rotation
 *       and a V deviation share one launch.
 *   CB_ORDER_SELECT_FIRST : score (V only), select, then cb_rerotate_fuse:
 *       the rows of S are written once and never re-rotated.
 *   CB_ORDER_AUTO : select first for a V deviation when the layer's K cache
 *       (n_tok rows) is at most CB_SELECT_FIRST_MAX_BYTES, or when the shared
 *       launch does not cover the geometry; rotate first otherwise.  Where
 *       the re-rotation is long it hides the deviation in the shared launch;
 *       where it is short, saving the bytes of S and a smaller first launch
 *       win.  Either order gives the same results bit for bit. */
typedef enum {
  CB_ORDER_AUTO = 0,
  CB_ORDER_ROTATE_FIRST = 1,
  CB_ORDER_SELECT_FIRST = 2
} cb_order;
#define CB_SELECT_FIRST_MAX_BYTES (16u << 20)

/* Every argument of one layer of the blend. */
typedef struct cb_layer_args {
  cb_geom geom;
  cb_ragged rg;
  void *k;              /* [T][Hkv][D] cached K: re-rotated, then fused, in place */
  void *v;              /* [T][Hkv][D] cached V: fused in place */
  const void *k_new_c;  /* [M][Hkv][D] */
  const void *v_new_c;  /* [M][Hkv][D] */
  const void *q_c;      /* [M][Hq][D] */
  const int32_t *delta; /* [T] p_new - p_old; NULL = keys already at p_new */
  const int32_t *cand_idx; /* [M] */
  double rope_theta;
  int32_t rope_style;
  float softmax_scale;
  float *dev;           /* [M] out */
  int32_t *sel_local;   /* [K] out */
  int32_t *sel_global;  /* [K] out */
  void *out;            /* [K][Hq][D] out */
  void *workspace;      /* optional attention workspace (see cb_partial_attn) */
  size_t workspace_bytes;
  int32_t dev_source;   /* cb_dev_source; CB_DEV_V is the score of [Derivations] */
  int32_t order;        /* a cb_order value; 0 is CB_ORDER_AUTO */
  uint32_t flags;       /* 0 or CB_LAYER_WORKSPACE_ZEROED (other bits: INVALID_ARG) */
} cb_layer_args;

/* cb_layer_args.flags: the caller filled the workspace with zeros before its
 * first use by cb_blend_layer and has used it since only for cb_blend_layer
 * calls.  The last CB_SELECT_COUNTER_BYTES of the workspace then hold one
 * arrival counter per request, which every call leaves at zero, and for a V
 * deviation with at most CB_SELECT_COUNTER_BYTES / 4 requests the top-k runs
 * inside the deviation launch (the workgroup that scores a request's last
 * candidates selects its rows): one launch fewer per layer, the same results
 * bit for bit.  The attention then uses the workspace without those bytes.
 * Ignored with a workspace smaller than CB_SELECT_COUNTER_BYTES.  Counters
 * that are not zero give wrong selections (a request selected before all of
 * its scores are written, or never); nothing waits on them, so nothing hangs. */
#define CB_LAYER_WORKSPACE_ZEROED 1u
#define CB_SELECT_COUNTER_BYTES 4096u

/*
 * cb_blend_layer -- one layer: cb_rerotate (in place, when delta != NULL) ->
 * cb_kv_deviation_topk (keys scored after their re-rotation) ->
 * cb_fuse_scatter -> cb_partial_attn, all on `stream` (with
 * CB_LAYER_WORKSPACE_ZEROED the deviation and the top-k share one launch).  With the order
 * CB_ORDER_SELECT_FIRST (or CB_ORDER_AUTO choosing it): cb_kv_deviation_topk
 * (V) -> cb_rerotate_fuse -> cb_partial_attn, with the same results bit for
 * bit (INVALID_ARG for CB_ORDER_SELECT_FIRST with a key deviation source,
 * which needs the keys re-rotated before it).
 * [KV-blog, "渐进式过滤机制"]: the caller runs it per layer, passing all
 * tokens as candidates at layer 1 and the surviving rows afterwards.
 * Precondition (not checked on the host): cand_idx is ascending within each
 * request and the requests' rows follow each other, so that the selection
 * (cand_idx[sel_local]) is strictly ascending over the whole batch, as the
 * rotate-or-replace pass of CB_ORDER_SELECT_FIRST requires.  With candidates
 * out of order that pass may turn a selected row instead of replacing it;
 * the selection written by a previous layer's call always qualifies.
 */
cb_status cb_blend_layer(const cb_layer_args *args, void *stream);

/* The order cb_blend_layer follows for these arguments
 * (CB_ORDER_ROTATE_FIRST or CB_ORDER_SELECT_FIRST), after the same checks of
 * the order field; host only, enqueues nothing. */
cb_status cb_blend_layer_order(const cb_layer_args *args, int32_t *order);

/*
 * cb_blend_layer_noalloc -- cb_blend_layer for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, steps and results as
 * cb_blend_layer, except that args->workspace must be NULL and
 * args->workspace_bytes 0 (else CB_ERR_INVALID_ARG): the attention's split
 * partials and arrival counters live in a static device array of the library
 * of CB_NOALLOC_SCRATCH_BYTES, one per GPU, held from the library's first use
 * on that GPU until the process ends.  Long rows are split only by plans
 * that fit in it, less its last CB_SELECT_COUNTER_BYTES (where cb_blend_layer with a larger workspace would split
 * further, this call keeps the best plan that fits, or none; outputs then
 * agree to rounding, selections and fused rows bit for bit); a plan larger
 * than the array is refused with CB_ERR_UNSUPPORTED before anything is
 * enqueued.  The array starts zero-filled, so the call always runs the top-k
 * inside the deviation launch as CB_LAYER_WORKSPACE_ZEROED describes (its
 * last CB_SELECT_COUNTER_BYTES hold those counters; args->flags may be 0 or
 * that flag).  The call allocates and frees nothing; its first call on a GPU
 * looks up the array's device address there (a HIP symbol query).
 * The array keeps the last call's contents; each call clears the attention
 * counters it uses in its own fuse launch and leaves the selection counters
 * at zero.  Every call in a process shares the GPU's one
 * array, so calls that may overlap on one GPU (different streams or host
 * threads) race: order them, e.g. on one stream.
 */
#define CB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
cb_status cb_blend_layer_noalloc(const cb_layer_args *args, void *stream);

/*
 * cb_check_indices -- checks on the device the index preconditions that the
 * other calls do not check on the host (they would cost a device read):
 *   CB_CHECK_CAND_RANGE    1  a cand_idx entry of request r lies outside
 *                             [tok_off[r], tok_off[r+1])
 *   CB_CHECK_CAND_ORDER    2  cand_idx does not ascend strictly within a request
 *   CB_CHECK_SEL_RANGE     4  a sel_global entry lies outside its request's rows
 *   CB_CHECK_SEL_ORDER     8  sel_global does not ascend strictly over the whole
 *                             batch (cb_rerotate_fuse and CB_ORDER_SELECT_FIRST
 *                             rely on it; a previous layer's selection always
 *                             qualifies)
 *   CB_CHECK_LOCAL_RANGE  16  a sel_local entry lies outside its request's
 *                             candidate range
 *   CB_CHECK_LOCAL_MISMATCH 32  cand_idx[sel_local[s]] != sel_global[s]
 *
 *   rg          : the ragged batch (tok_off, cand_off, sel_off on the device
 *                 and their host mirrors; cand_off may be NULL when cand_idx
 *                 and sel_local are)
 *   cand_idx    : [M] or NULL (its checks skipped)
 *   sel_local, sel_global : [K] or NULL (their checks skipped)
 *   flags       : device int32, written with the OR of the violations found
 *                 (0: every check passed); no clearing needed beforehand.
 * One workgroup, stream-ordered, no allocation: a debugging aid, also safe
 * under graph capture.  Errors: INVALID_ARG for a NULL flags or invalid
 * offsets, before any HIP call.
 */
#define CB_CHECK_CAND_RANGE 1
#define CB_CHECK_CAND_ORDER 2
#define CB_CHECK_SEL_RANGE 4
#define CB_CHECK_SEL_ORDER 8
#define CB_CHECK_LOCAL_RANGE 16
#define CB_CHECK_LOCAL_MISMATCH 32
cb_status cb_check_indices(const cb_ragged *rg, const int32_t *cand_idx,
                           const int32_t *sel_local, const int32_t *sel_global, int32_t *flags,
                           void *stream);

/* Static description of a status code. */
const char *cb_status_str(cb_status status);
/* Detail text of the calling thread's last failing call ("" if none). */
const char *cb_last_error(void);
/* ABI revision of this header (bumped on any incompatible change). */
int32_t cb_abi_version(void);

#define CB_ABI_VERSION 7

#ifdef __cplusplus
}
#endif

#endif /* CACHEBLEND_H */

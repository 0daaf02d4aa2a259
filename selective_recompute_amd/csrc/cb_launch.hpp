// Internal launcher interface between the C ABI (api.cpp) and the kernels.
// Every launcher enqueues on `stream` and returns the launch status; none of
// them validates arguments (api.cpp does that before calling).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cb {

// Turning speed of each RoPE pair in revolutions per position:
// omega_j / (2 pi), omega_j = theta^(-2j/D), computed on the host in double.
struct RopeTable {
  double rev_per_pos[64];
};

enum : int { kF32 = 0, kBF16 = 1 };

hipError_t launch_rerotate(int dtype, int style, void *k_out, const void *k_in,
                           const int32_t *delta, int64_t n_tok, int32_t n_layers,
                           int32_t n_kv_heads, int32_t head_dim,
                           const RopeTable &tab, hipStream_t stream);

// Re-rotation (in place, one layer) and deviation fused in one launch; only
// for geometries where a re-rotation row fits a 256-thread workgroup.
bool rerotate_deviation_fits(int dtype, int32_t n_kv_heads, int32_t head_dim);
hipError_t launch_rerotate_deviation(int dtype, int style, void *k, const int32_t *delta,
                                     int64_t n_tok, int32_t n_kv_heads, int32_t head_dim,
                                     const RopeTable &tab, const void *v_new_c,
                                     const void *v_old, const int32_t *cand_idx, float *dev,
                                     int64_t m, hipStream_t stream);

// dev[j] = squared distance of row j of new0 and row cand_idx[j] of old0,
// plus the same for new1 / old1 when new1 is not NULL (the K and V rows of a
// token read as one vector).
hipError_t launch_deviation(int dtype, const void *new0, const void *old0, const void *new1,
                            const void *old1, const int32_t *cand_idx, float *dev, int64_t m,
                            int32_t row_elems, hipStream_t stream);

// h_cand_off / h_sel_off: host mirrors of the offsets (grid sizing; a single
// request's counts also travel as kernel arguments).
hipError_t launch_topk(int32_t n_req, const float *dev, const int32_t *cand_idx,
                       const int32_t *cand_off, const int32_t *sel_off, int32_t *sel_local,
                       int32_t *sel_global, const int32_t *h_cand_off, const int32_t *h_sel_off,
                       hipStream_t stream);

// V deviation and top-k in one launch; with k != NULL the same launch also
// re-rotates K in place (only where rerotate_deviation_fits).  cnt: one
// arrival counter per request, zero before the launch and left at zero by
// it.  h_cand_off: host mirror (grid and register-path sizing).
constexpr int kSelectMaxRequests = 1024;  // counters in CB_SELECT_COUNTER_BYTES
hipError_t launch_deviation_select(int dtype, int style, void *k, const int32_t *delta,
                                   int64_t n_tok, int32_t n_kv_heads, int32_t head_dim,
                                   const RopeTable &tab, const void *v_new_c, const void *v_old,
                                   const int32_t *cand_idx, float *dev, int32_t n_req,
                                   const int32_t *cand_off, const int32_t *sel_off,
                                   const int32_t *h_cand_off, int32_t *sel_local,
                                   int32_t *sel_global, unsigned *cnt, hipStream_t stream);

// Device-side check of the index preconditions (one workgroup); writes the
// violation bits to *flags.  cand_idx / sel_local / sel_global may be NULL.
hipError_t launch_check_indices(const int32_t *tok_off, const int32_t *cand_off,
                                const int32_t *sel_off, int32_t n_req, const int32_t *cand_idx,
                                const int32_t *sel_local, const int32_t *sel_global,
                                int32_t *flags, hipStream_t stream);

// Also sets clear[0 .. n_clear) to zero (the attention's arrival counters;
// clear may be NULL when n_clear is 0).
hipError_t launch_fuse(void *k_fused, void *v_fused, const void *k_new_c,
                       const void *v_new_c, const int32_t *sel_local,
                       const int32_t *sel_global, int64_t k_total,
                       int32_t row_bytes, uint32_t *clear, int64_t n_clear,
                       hipStream_t stream);

// Rotate-or-replace after the selection (rows of S take the new K/V rows,
// every other row's K is re-rotated by delta); also zeroes clear[0 .. n_clear).
// sel_global ascending.
hipError_t launch_rerotate_fuse(int dtype, int style, void *k, void *v, const void *k_new_c,
                                const void *v_new_c, const int32_t *delta,
                                const int32_t *sel_local, const int32_t *sel_global,
                                int64_t k_total, int64_t n_tok, int32_t n_kv_heads,
                                int32_t head_dim, const RopeTable &tab, uint32_t *clear,
                                int64_t n_clear, hipStream_t stream);

// Partial attention.
struct AttnArgs {
  void *out;
  const void *q_c;
  const int32_t *sel_local;
  const int32_t *sel_global;
  const void *k_fused;
  const void *v_fused;
  const int32_t *tok_off;
  const int32_t *sel_off;
  const int32_t *h_tok_off;  // host mirrors of tok_off / sel_off (launch order)
  const int32_t *h_sel_off;
  void *workspace;
  int32_t n_req;
  int32_t k_total;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  float softmax_scale;
};

// Host-side decomposition of the MFMA attention launch.
struct AttnPlan {
  int key_split;       // key groups per workgroup (1: 256, 2: 128 query vectors per tile)
  int rows_per_tile;   // selected rows per query tile
  int key_chunk;       // keys per unit (multiple of the 64 * key_split keys of a tile); huge = no split
  bool split;          // some request has more than one chunk
  int64_t tiles;       // query tiles over all requests
  int64_t units;       // (tile, chunk) units over all requests
  size_t cnt_offset;   // split: byte offset of the arrival counters in the workspace
  int64_t n_cnt;       // split: arrival counters, one per (tile, KV head)
  size_t ws_bytes;     // workspace the split needs: partials, then counters
  int spans;           // > 0: balanced decomposition (key split 1): the 64-key tiles of
                       // all query tiles of a KV head cut into `spans` equal spans, one
                       // workgroup each (units = spans); 0: (tile, key chunk) units
};

// Selected rows per MFMA query tile (256 / key_split query vectors), or 0 if
// the MFMA kernel does not cover this geometry with that key split (1 or 2).
int attn_mfma_rows_per_tile(int dtype, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, int key_split);
// Workspace bytes of one split unit.
size_t attn_unit_bytes(int32_t head_dim, int key_split);
// Most key chunks one row may be split into.
int attn_max_chunks();
// Whether a batch fits the balanced decomposition's tables (requests, query tiles).
bool attn_stream_fits(int32_t n_req, int64_t tiles);

// Most units whose launch order the host can choose (a table in the kernel
// arguments); unsplit plans, plans with more units and the balanced
// decomposition run in the kernel's own order.
constexpr int kAttnMaxOrder = 960;

// counters_zero: the split's arrival counters are already zero (cleared by
// the preceding fuse launch); otherwise a clear launch goes first.
hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &plan, bool counters_zero,
                            hipStream_t stream);

hipError_t launch_attn_simple(int dtype, const AttnArgs &a, hipStream_t stream);

// The library's own device scratch (scratch.hip): the attention workspace of
// cb_blend_layer_noalloc.  noalloc_scratch() gives its address on the
// current device (looked up once per device); it allocates nothing.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);

}  // namespace cb

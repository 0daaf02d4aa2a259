// extern "C" entry points of libcacheblend: host-side validation, then the
// kernel launches.  Validation makes no HIP call, so every argument error is
// reported synchronously with nothing enqueued.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <queue>
#include <string>
#include <vector>

#include "cacheblend.h"
#include "cb_launch.hpp"

#define CB_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

cb_status fail(cb_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t dtype) { return dtype == CB_DTYPE_BF16 ? 2 : 4; }

#define CB_TRY(expr)                 \
  do {                               \
    cb_status _st = (expr);          \
    if (_st != CB_OK) return _st;    \
  } while (0)

cb_status check_geom(const cb_geom *g) {
  if (!g) return fail(CB_ERR_INVALID_ARG, "geom is NULL");
  if (g->dtype != CB_DTYPE_F32 && g->dtype != CB_DTYPE_BF16)
    return fail(CB_ERR_UNSUPPORTED, "dtype %d is not CB_DTYPE_F32 or CB_DTYPE_BF16", g->dtype);
  if (g->n_kv_heads < 1 || g->n_q_heads < 1)
    return fail(CB_ERR_INVALID_ARG, "head counts must be >= 1 (q %d, kv %d)", g->n_q_heads,
                g->n_kv_heads);
  if (g->n_q_heads % g->n_kv_heads != 0)
    return fail(CB_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d",
                g->n_q_heads, g->n_kv_heads);
  if (g->head_dim != 16 && g->head_dim != 32 && g->head_dim != 64 && g->head_dim != 128)
    return fail(CB_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", g->head_dim);
  // one rerotate unit per 16 bytes of half a head; a row must fit a workgroup
  const int pairs_per_unit = 16 / elem_size(g->dtype);
  const int64_t units = (int64_t)g->n_kv_heads * (g->head_dim / 2) / pairs_per_unit;
  if (units > 1024)
    return fail(CB_ERR_UNSUPPORTED, "n_kv_heads %d too large for head_dim %d", g->n_kv_heads,
                g->head_dim);
  if (g->n_q_heads > 65535) return fail(CB_ERR_UNSUPPORTED, "n_q_heads too large");
  return CB_OK;
}

cb_status need_ptr(const void *p, const char *name, bool needed) {
  if (!needed) return CB_OK;
  if (!p) return fail(CB_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(CB_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return CB_OK;
}

cb_status need_idx(const void *p, const char *name, bool needed) {
  if (!needed) return CB_OK;
  if (!p) return fail(CB_ERR_INVALID_ARG, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0)
    return fail(CB_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
  return CB_OK;
}

cb_status check_offsets(const int32_t *h, int32_t n, const char *name) {
  if (!h) return fail(CB_ERR_INVALID_ARG, "host mirror %s is NULL", name);
  if (h[0] != 0) return fail(CB_ERR_INVALID_ARG, "%s[0] = %d, expected 0", name, h[0]);
  for (int32_t r = 0; r < n; ++r)
    if (h[r + 1] < h[r])
      return fail(CB_ERR_INVALID_ARG, "%s decreases at request %d", name, r);
  return CB_OK;
}

// Ragged batch checks.  want_tok/want_cand/want_sel: which offsets the call uses.
cb_status check_ragged(const cb_ragged *rg, bool want_tok, bool want_cand, bool want_sel) {
  if (!rg) return fail(CB_ERR_INVALID_ARG, "ragged descriptor is NULL");
  if (rg->n_req < 1) return fail(CB_ERR_INVALID_ARG, "n_req %d < 1", rg->n_req);
  if (want_tok) {
    CB_TRY(need_idx(rg->tok_off, "tok_off", true));
    CB_TRY(check_offsets(rg->h_tok_off, rg->n_req, "h_tok_off"));
  }
  if (want_cand) {
    CB_TRY(need_idx(rg->cand_off, "cand_off", true));
    CB_TRY(check_offsets(rg->h_cand_off, rg->n_req, "h_cand_off"));
  }
  if (want_sel) {
    CB_TRY(need_idx(rg->sel_off, "sel_off", true));
    CB_TRY(check_offsets(rg->h_sel_off, rg->n_req, "h_sel_off"));
  }
  for (int32_t r = 0; r < rg->n_req; ++r) {
    const int64_t n = want_tok ? (int64_t)rg->h_tok_off[r + 1] - rg->h_tok_off[r] : -1;
    const int64_t m = want_cand ? (int64_t)rg->h_cand_off[r + 1] - rg->h_cand_off[r] : -1;
    const int64_t k = want_sel ? (int64_t)rg->h_sel_off[r + 1] - rg->h_sel_off[r] : -1;
    if (want_cand && want_sel && k > m)
      return fail(CB_ERR_INVALID_ARG, "request %d selects %lld of %lld candidates", r,
                  (long long)k, (long long)m);
    if (want_tok && want_cand && m > n)
      return fail(CB_ERR_INVALID_ARG, "request %d has %lld candidates for %lld tokens", r,
                  (long long)m, (long long)n);
    if (want_tok && want_sel && k > n)
      return fail(CB_ERR_INVALID_ARG, "request %d selects %lld rows of %lld tokens", r,
                  (long long)k, (long long)n);
  }
  return CB_OK;
}

cb_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return CB_OK;
  return fail(CB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t row_elems(const cb_geom *g) { return (int64_t)g->n_kv_heads * g->head_dim; }

cb_status validate_rerotate(const cb_geom *geom, void *k_out, const void *k_in,
                            const int32_t *delta, int64_t n_tok, int32_t n_layers,
                            double rope_theta, int32_t rope_style) {
  CB_TRY(check_geom(geom));
  if (n_tok < 0 || n_tok >= INT32_MAX) return fail(CB_ERR_INVALID_ARG, "n_tok %lld out of range", (long long)n_tok);
  if (n_layers < 1) return fail(CB_ERR_INVALID_ARG, "n_layers %d < 1", n_layers);
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(CB_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (rope_style != CB_ROPE_HALF && rope_style != CB_ROPE_INTERLEAVED)
    return fail(CB_ERR_INVALID_ARG, "rope_style %d unknown", rope_style);
  const bool any = n_tok > 0;
  CB_TRY(need_ptr(k_in, "k_in", any));
  CB_TRY(need_ptr(k_out, "k_out", any));
  CB_TRY(need_idx(delta, "delta", any));
  if (any && k_out != k_in) {
    const int64_t bytes = (int64_t)n_layers * n_tok * row_elems(geom) * elem_size(geom->dtype);
    const char *a = static_cast<const char *>(k_in), *b = static_cast<const char *>(k_out);
    if (a < b + bytes && b < a + bytes)
      return fail(CB_ERR_INVALID_ARG, "k_out partially overlaps k_in");
  }
  return CB_OK;
}

cb::RopeTable rope_table(int head_dim, double theta) {
  cb::RopeTable t{};
  const double two_pi = 6.283185307179586476925;
  for (int j = 0; j < head_dim / 2; ++j)
    t.rev_per_pos[j] = std::pow(theta, -2.0 * j / head_dim) / two_pi;
  return t;
}

cb_status validate_devtopk(const cb_geom *geom, const cb_ragged *rg, int32_t source,
                           const void *k_new_c, const void *k_cached, const void *v_new_c,
                           const void *v_old, const int32_t *cand_idx, const float *dev,
                           const int32_t *sel_local, const int32_t *sel_global) {
  CB_TRY(check_geom(geom));
  CB_TRY(check_ragged(rg, true, true, true));
  if (source != CB_DEV_V && source != CB_DEV_K && source != CB_DEV_KV)
    return fail(CB_ERR_INVALID_ARG, "deviation source %d unknown", source);
  const int32_t m = rg->h_cand_off[rg->n_req], k = rg->h_sel_off[rg->n_req];
  const bool uses_k = source != CB_DEV_V, uses_v = source != CB_DEV_K;
  CB_TRY(need_ptr(k_new_c, "k_new_c", m > 0 && uses_k));
  CB_TRY(need_ptr(k_cached, "k_cached", m > 0 && uses_k));
  CB_TRY(need_ptr(v_new_c, "v_new_c", m > 0 && uses_v));
  CB_TRY(need_ptr(v_old, "v_old", m > 0 && uses_v));
  CB_TRY(need_idx(cand_idx, "cand_idx", m > 0));
  CB_TRY(need_idx(dev, "dev", m > 0));
  CB_TRY(need_idx(sel_local, "sel_local", k > 0));
  CB_TRY(need_idx(sel_global, "sel_global", k > 0));
  return CB_OK;
}

// The deviation launch of a validated source: one tensor pair, or K then V.
hipError_t launch_dev_source(const cb_geom *geom, int32_t source, const void *k_new_c,
                             const void *k_cached, const void *v_new_c, const void *v_old,
                             const int32_t *cand_idx, float *dev, int64_t m, hipStream_t s) {
  const int32_t re = (int32_t)row_elems(geom);
  if (source == CB_DEV_V)
    return cb::launch_deviation(geom->dtype, v_new_c, v_old, nullptr, nullptr, cand_idx, dev, m,
                                re, s);
  if (source == CB_DEV_K)
    return cb::launch_deviation(geom->dtype, k_new_c, k_cached, nullptr, nullptr, cand_idx, dev,
                                m, re, s);
  return cb::launch_deviation(geom->dtype, k_new_c, k_cached, v_new_c, v_old, cand_idx, dev, m,
                              re, s);
}

cb_status validate_topk(const cb_ragged *rg, const float *dev, const int32_t *cand_idx,
                        const int32_t *sel_local, const int32_t *sel_global) {
  CB_TRY(check_ragged(rg, false, true, true));
  const int32_t m = rg->h_cand_off[rg->n_req], k = rg->h_sel_off[rg->n_req];
  CB_TRY(need_idx(dev, "dev", m > 0));
  CB_TRY(need_idx(cand_idx, "cand_idx", m > 0));
  CB_TRY(need_idx(sel_local, "sel_local", k > 0));
  CB_TRY(need_idx(sel_global, "sel_global", k > 0));
  return CB_OK;
}

cb_status validate_fuse(const cb_geom *geom, void *k_fused, void *v_fused, const void *k_new_c,
                        const void *v_new_c, const int32_t *sel_local, const int32_t *sel_global,
                        int64_t k_total) {
  CB_TRY(check_geom(geom));
  if (k_total < 0 || k_total >= INT32_MAX) return fail(CB_ERR_INVALID_ARG, "k_total out of range");
  const bool any = k_total > 0;
  CB_TRY(need_ptr(k_fused, "k_fused", any));
  CB_TRY(need_ptr(v_fused, "v_fused", any));
  CB_TRY(need_ptr(k_new_c, "k_new_c", any));
  CB_TRY(need_ptr(v_new_c, "v_new_c", any));
  CB_TRY(need_idx(sel_local, "sel_local", any));
  CB_TRY(need_idx(sel_global, "sel_global", any));
  return CB_OK;
}

cb_status validate_attn(const cb_geom *geom, const cb_ragged *rg, void *out, const void *q_c,
                        const int32_t *sel_local, const int32_t *sel_global, const void *k_fused,
                        const void *v_fused, float softmax_scale) {
  CB_TRY(check_geom(geom));
  CB_TRY(check_ragged(rg, true, false, true));
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CB_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  const int32_t k = rg->h_sel_off[rg->n_req];
  const bool any = k > 0;
  CB_TRY(need_ptr(out, "out", any));
  CB_TRY(need_ptr(q_c, "q_c", any));
  CB_TRY(need_ptr(k_fused, "k_fused", any));
  CB_TRY(need_ptr(v_fused, "v_fused", any));
  CB_TRY(need_idx(sel_local, "sel_local", any));
  CB_TRY(need_idx(sel_global, "sel_global", any));
  if ((int64_t)k * geom->n_q_heads > INT32_MAX)
    return fail(CB_ERR_UNSUPPORTED, "k_total * n_q_heads exceeds the grid limit");
  return CB_OK;
}

constexpr int kNoSplit = 1 << 30;

// Cost model of one MFMA attention launch, for choosing the key split and
// the key chunk.  The figures are in microseconds at head_dim 128 (they
// scale with head_dim), fitted on MI355X to the measured best plans of the
// 2k-, 6k- and 32k-token single-request shapes over key splits and chunk
// sizes: 64 keys of a 256-query unit take ~1.6 us on a lightly loaded chip,
// and kKeySplitTile of that for a 128-query unit whose 128-key tiles are
// split over two wave groups; a workgroup spends ~3.6 us before its first
// tile (three dependent loads: request offsets, selected rows, Q) and, when
// split, ~5 us storing its partial at the coherence point and signalling;
// the last working unit of a split tile then spends kMergeUs arriving plus
// kMergePairUs per two other partials it loads and merges.
constexpr double kTileUs = 1.6, kSetupUs = 3.6, kPartialUs = 5.0;
constexpr double kKeySplitTile = 0.55;
constexpr double kMergeUs = 1.0, kMergePairUs = 1.0;
// CUs the simulated dispatch fills: 240 of the 256, a margin against plans
// that fit one more round only if the selected rows sit exactly as assumed.
constexpr int kSimCUs = 240;

// Estimated duration (us) of the launch with key split `ks`, `rows` selected
// rows per tile and key chunk `kc` (kNoSplit: none), and the number of units
// that do work.  The selected rows of a request are taken as evenly spread
// over its tokens, so query tile t ends near position min(k, (t+1) rows) n / k.
// Units are dispatched in launch order, each to the earliest free group of
// CUs: longest unit first where cb::launch_attn_mfma orders the launch
// (split plans of up to cb::kAttnMaxOrder units), else the kernel's own
// order (request by request, chunk by chunk, longest tile first).  The n_kv_heads workgroups of a unit run side by side, so one
// "slot" stands for n_kv_heads CUs.  A split tile ends when its last unit
// has merged.
double estimate_attn_us(const cb_geom *g, const cb_ragged *rg, int ks, int rows, int64_t kc,
                        int64_t *active) {
  const int n_slots = std::max(1, kSimCUs / g->n_kv_heads);
  const double tile_us = kTileUs * g->head_dim / 128.0 * (ks == 2 ? kKeySplitTile : 1.0);
  const double partial_us = kPartialUs / ks;
  const int64_t kt = 64 * ks;  // keys per tile
  struct Unit { double us; int64_t tile; };  // tile: index over all requests
  std::vector<Unit> units;
  std::vector<int> tile_units;
  int64_t tbase = 0, all_units = 0;
  bool split = false;
  for (int32_t r = 0; r < rg->n_req; ++r) {
    const int64_t k = rg->h_sel_off[r + 1] - rg->h_sel_off[r];
    const int64_t n = rg->h_tok_off[r + 1] - rg->h_tok_off[r];
    if (k == 0) continue;
    const int64_t tiles = (k + rows - 1) / rows;
    const int64_t chunks = (n + kc - 1) / kc;
    all_units += tiles * chunks;
    if (chunks > 1) split = true;
    tile_units.resize((size_t)(tbase + tiles), 0);
    for (int64_t c = 0; c < chunks; ++c)
      for (int64_t t = tiles - 1; t >= 0; --t) {
        const int64_t end = (std::min(k, (t + 1) * rows) * n + k - 1) / k;
        const int64_t lo = c * kc, hi = std::min(end, lo + kc);
        if (hi <= lo) continue;
        const double us = kSetupUs + (double)((hi - lo + kt - 1) / kt * ks) * tile_us +
                          (chunks > 1 ? partial_us : 0.0);
        units.push_back({us, tbase + t});
        ++tile_units[(size_t)(tbase + t)];
      }
    tbase += tiles;
  }
  if (split && all_units <= cb::kAttnMaxOrder)
    std::stable_sort(units.begin(), units.end(),
                     [](const Unit &x, const Unit &y) { return x.us > y.us; });
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < n_slots; ++i) free_at.push(0.0);
  std::vector<double> tile_end((size_t)tbase, 0.0);
  for (const Unit &u : units) {
    const double start = free_at.top();
    free_at.pop();
    free_at.push(start + u.us);
    tile_end[(size_t)u.tile] = std::max(tile_end[(size_t)u.tile], start + u.us);
  }
  double makespan = 0.0;
  for (int64_t t = 0; t < tbase; ++t) {
    const int u = tile_units[(size_t)t];
    const double merge = u > 1 ? kMergeUs + (double)(u / 2) * kMergePairUs : 0.0;
    makespan = std::max(makespan, tile_end[(size_t)t] + merge);
  }
  *active = (int64_t)units.size();
  return makespan;
}

// Workspace of a split: the partials of every workgroup, then (256-byte
// aligned) one arrival counter per (tile, KV head).
size_t split_ws_bytes(const cb_geom *g, int ks, int64_t units, int64_t tiles,
                      size_t *cnt_offset = nullptr) {
  const size_t partials = (size_t)units * g->n_kv_heads * cb::attn_unit_bytes(g->head_dim, ks);
  const size_t off = (partials + 255) / 256 * 256;
  if (cnt_offset) *cnt_offset = off;
  return off + (size_t)tiles * g->n_kv_heads * sizeof(uint32_t);
}

// Workspace of the balanced decomposition: two partial slots per workgroup,
// then (256-byte aligned) one arrival counter per (query tile, KV head).
size_t stream_ws_bytes(const cb_geom *g, int spans, int64_t tiles, size_t *cnt_offset = nullptr) {
  const size_t partials =
      (size_t)spans * g->n_kv_heads * 2 * cb::attn_unit_bytes(g->head_dim, 1);
  const size_t off = (partials + 255) / 256 * 256;
  if (cnt_offset) *cnt_offset = off;
  return off + (size_t)tiles * g->n_kv_heads * sizeof(uint32_t);
}

// Fills the counts of an MFMA plan whose key split, rows per tile and key
// chunk (or spans) are set: tiles, units, split, counters, workspace.
void finish_plan(const cb_geom *g, const cb_ragged *rg, cb::AttnPlan &pl) {
  const int rows = pl.rows_per_tile;
  pl.tiles = pl.units = 0;
  pl.split = false;
  if (pl.spans > 0) {
    for (int32_t r = 0; r < rg->n_req; ++r)
      pl.tiles += (rg->h_sel_off[r + 1] - rg->h_sel_off[r] + rows - 1) / rows;
    pl.units = pl.spans;
    pl.split = pl.tiles > 0;
    pl.n_cnt = pl.split ? pl.tiles * g->n_kv_heads : 0;
    pl.ws_bytes = pl.split ? stream_ws_bytes(g, pl.spans, pl.tiles, &pl.cnt_offset) : 0;
    return;
  }
  for (int32_t r = 0; r < rg->n_req; ++r) {
    const int64_t kr = rg->h_sel_off[r + 1] - rg->h_sel_off[r];
    const int64_t n = rg->h_tok_off[r + 1] - rg->h_tok_off[r];
    const int64_t tr = (kr + rows - 1) / rows;
    const int64_t cr = (n + pl.key_chunk - 1) / pl.key_chunk;
    pl.tiles += tr;
    pl.units += tr * cr;
    if (tr > 0 && cr > 1) pl.split = true;
  }
  pl.cnt_offset = 0;
  pl.n_cnt = pl.split ? pl.tiles * g->n_kv_heads : 0;
  pl.ws_bytes = pl.split ? split_ws_bytes(g, pl.key_split, pl.units, pl.tiles, &pl.cnt_offset) : 0;
}

// Decomposition of the MFMA attention, from host mirrors only (never the
// balanced decomposition, which only a pinned plan selects: on the shapes
// measured its cut pieces cost more than its balance gains).  When the
// query tiles of 256 query vectors give 1024 workgroups or more, that is the
// plan.  Otherwise the cost model above picks, among the plans whose
// workspace fits in `ws_avail`, the shortest of: key split 1 or 2 (2 only
// when its working workgroups fit on the CUs at once), each either unsplit
// or with long rows split over key chunks (a multiple of the tile, 64 or 128
// keys, at least 256, at most attn_max_chunks() per request).
cb::AttnPlan plan_attn(const cb_geom *g, const cb_ragged *rg, size_t ws_avail) {
  cb::AttnPlan pl{};
  pl.key_split = 1;
  pl.key_chunk = kNoSplit;
  pl.rows_per_tile = cb::attn_mfma_rows_per_tile(g->dtype, g->n_q_heads, g->n_kv_heads,
                                                 g->head_dim, 1);
  if (pl.rows_per_tile == 0) return pl;
  auto count_tiles = [&](int rows) {
    int64_t tiles = 0;
    for (int32_t r = 0; r < rg->n_req; ++r)
      tiles += (rg->h_sel_off[r + 1] - rg->h_sel_off[r] + rows - 1) / rows;
    return tiles;
  };
  auto count_units = [&](int rows, int64_t kc, bool &split) {
    int64_t units = 0;
    split = false;
    for (int32_t r = 0; r < rg->n_req; ++r) {
      const int64_t kr = rg->h_sel_off[r + 1] - rg->h_sel_off[r];
      const int64_t n = rg->h_tok_off[r + 1] - rg->h_tok_off[r];
      const int64_t tr = (kr + rows - 1) / rows;
      const int64_t cr = (n + kc - 1) / kc;
      units += tr * cr;
      if (tr > 0 && cr > 1) split = true;
    }
    return units;
  };
  int64_t max_n = 0;
  for (int32_t r = 0; r < rg->n_req; ++r)
    if (rg->h_sel_off[r + 1] > rg->h_sel_off[r])
      max_n = std::max<int64_t>(max_n, rg->h_tok_off[r + 1] - rg->h_tok_off[r]);
  const int64_t blocks = count_tiles(pl.rows_per_tile) * g->n_kv_heads;
  if (blocks > 0 && blocks < 1024) {
    int64_t active = 0;
    double best = estimate_attn_us(g, rg, 1, pl.rows_per_tile, kNoSplit, &active);
    auto consider = [&](int ks, int rows, int64_t kc) {
      bool split = false;
      const int64_t units = count_units(rows, kc, split);
      const size_t ws = split ? split_ws_bytes(g, ks, units, count_tiles(rows)) : 0;
      if (ws > ws_avail) return;
      const double us = estimate_attn_us(g, rg, ks, rows, kc, &active);
      // Key split 2 only where its working units fit in one round of the CUs:
      // there the shorter units decide; with more rounds its ~5% higher cost
      // per flop and its doubled K/V reads through L2 decide against it (in
      // the full blend step: -4% at 2k tokens and one round, +1.5% at 6k
      // tokens and two rounds).
      if (ks == 2 && active * g->n_kv_heads > kSimCUs) return;
      if (us < best) {
        best = us;
        pl.key_split = ks;
        pl.rows_per_tile = rows;
        pl.key_chunk = (int)std::min<int64_t>(kc, kNoSplit);
      }
    };
    for (int ks = 1; ks <= 2; ++ks) {
      const int rows = cb::attn_mfma_rows_per_tile(g->dtype, g->n_q_heads, g->n_kv_heads,
                                                   g->head_dim, ks);
      if (rows == 0) continue;
      if (ks > 1) consider(ks, rows, kNoSplit);
      int64_t prev_kc = 0;
      for (int c = 2; c <= cb::attn_max_chunks(); ++c) {
        int64_t kc = (max_n + c - 1) / c;
        kc = std::max<int64_t>(256, (kc + 64 * ks - 1) / (64 * ks) * (64 * ks));
        if (kc >= max_n || kc == prev_kc) continue;
        prev_kc = kc;
        consider(ks, rows, kc);
      }
    }
  }
  finish_plan(g, rg, pl);
  return pl;
}

// A plan the caller pins (cb_partial_attn_with_plan): only mfma, key_split,
// key_chunk and stream_spans are read; the rest is derived as for a chosen plan.
cb_status pinned_plan(const cb_geom *g, const cb_ragged *rg, const cb_attn_plan *in,
                      size_t ws_avail, cb::AttnPlan &pl) {
  pl = cb::AttnPlan{};
  pl.key_split = 1;
  pl.key_chunk = kNoSplit;
  if (in->mfma == 0) return CB_OK;  // plain kernel: any geometry
  if (in->mfma != 1) return fail(CB_ERR_INVALID_ARG, "plan.mfma must be 0 or 1");
  if (in->key_split != 1 && in->key_split != 2)
    return fail(CB_ERR_INVALID_ARG, "plan.key_split must be 1 or 2");
  pl.key_split = in->key_split;
  pl.rows_per_tile = cb::attn_mfma_rows_per_tile(g->dtype, g->n_q_heads, g->n_kv_heads,
                                                 g->head_dim, pl.key_split);
  if (pl.rows_per_tile == 0)
    return fail(CB_ERR_UNSUPPORTED,
                "the MFMA kernel does not cover this geometry with key split %d (bf16, "
                "head_dim 32/64/128, a group size dividing %d query vectors)",
                pl.key_split, 256 / pl.key_split);
  const int tile_keys = 64 * pl.key_split;
  if (in->key_chunk < 0 || in->key_chunk % tile_keys != 0)
    return fail(CB_ERR_INVALID_ARG, "plan.key_chunk %d must be 0 or a positive multiple of %d",
                in->key_chunk, tile_keys);
  if (in->stream_spans < 0 || in->stream_spans > 65536)
    return fail(CB_ERR_INVALID_ARG, "plan.stream_spans %d must be in [0, 65536]",
                in->stream_spans);
  if (in->stream_spans > 0) {
    if (pl.key_split != 1 || in->key_chunk != 0)
      return fail(CB_ERR_INVALID_ARG,
                  "plan.stream_spans needs key_split 1 and key_chunk 0");
    pl.spans = in->stream_spans;
    finish_plan(g, rg, pl);
    if (!cb::attn_stream_fits(rg->n_req, pl.tiles))
      return fail(CB_ERR_UNSUPPORTED, "the balanced decomposition takes at most 1024 requests "
                  "and 2048 query tiles (%d requests, %lld tiles)", (int)rg->n_req,
                  (long long)pl.tiles);
    if (pl.ws_bytes > ws_avail)
      return fail(CB_ERR_INVALID_ARG, "workspace_bytes %zu is smaller than the plan's %zu",
                  ws_avail, pl.ws_bytes);
    return CB_OK;
  }
  if (in->key_chunk > 0) {
    pl.key_chunk = in->key_chunk;
    for (int32_t r = 0; r < rg->n_req; ++r) {
      const int64_t n = rg->h_tok_off[r + 1] - rg->h_tok_off[r];
      if (rg->h_sel_off[r + 1] > rg->h_sel_off[r] &&
          (n + pl.key_chunk - 1) / pl.key_chunk > cb::attn_max_chunks())
        return fail(CB_ERR_INVALID_ARG, "plan.key_chunk splits request %d into more than %d chunks",
                    (int)r, cb::attn_max_chunks());
    }
  }
  finish_plan(g, rg, pl);
  if (pl.ws_bytes > ws_avail)
    return fail(CB_ERR_INVALID_ARG, "workspace_bytes %zu is smaller than the plan's %zu",
                ws_avail, pl.ws_bytes);
  return CB_OK;
}

// counters_zero: the split's arrival counters in the workspace are known to
// be zero (cb_blend_layer's fuse launch clears them, or the caller vouches
// for them with CB_ATTN_COUNTERS_ZERO).
cb_status run_attn(const cb_geom *geom, const cb_ragged *rg, const cb::AttnPlan &plan,
                   void *out, const void *q_c, const int32_t *sel_local,
                   const int32_t *sel_global, const void *k_fused, const void *v_fused,
                   float softmax_scale, void *workspace, bool counters_zero,
                   hipStream_t stream) {
  cb::AttnArgs a;
  a.out = out; a.q_c = q_c; a.sel_local = sel_local; a.sel_global = sel_global;
  a.k_fused = k_fused; a.v_fused = v_fused; a.tok_off = rg->tok_off; a.sel_off = rg->sel_off;
  a.h_tok_off = rg->h_tok_off; a.h_sel_off = rg->h_sel_off;
  a.workspace = workspace;
  a.n_req = rg->n_req; a.k_total = rg->h_sel_off[rg->n_req];
  a.n_q_heads = geom->n_q_heads; a.n_kv_heads = geom->n_kv_heads; a.head_dim = geom->head_dim;
  a.softmax_scale = softmax_scale;
  if (a.k_total == 0) return CB_OK;
  if (plan.rows_per_tile > 0) {
    if (plan.units * geom->n_kv_heads > INT32_MAX)
      return fail(CB_ERR_UNSUPPORTED, "too many attention work units");
    return hip_status(cb::launch_attn_mfma(a, plan, counters_zero, stream), "partial_attn");
  }
  return hip_status(cb::launch_attn_simple(geom->dtype, a, stream), "partial_attn");
}

}  // namespace

CB_EXPORT cb_status cb_rerotate(const cb_geom *geom, void *k_out, const void *k_in,
                                const int32_t *delta, int64_t n_tok, int32_t n_layers,
                                double rope_theta, int32_t rope_style, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_rerotate(geom, k_out, k_in, delta, n_tok, n_layers, rope_theta, rope_style));
  if (n_tok == 0) return CB_OK;
  return hip_status(cb::launch_rerotate(geom->dtype, rope_style, k_out, k_in, delta, n_tok,
                                        n_layers, geom->n_kv_heads, geom->head_dim,
                                        rope_table(geom->head_dim, rope_theta),
                                        (hipStream_t)stream),
                    "rerotate");
}

CB_EXPORT cb_status cb_kv_deviation_topk(const cb_geom *geom, const cb_ragged *rg,
                                         int32_t source, const void *k_new_c,
                                         const void *k_cached, const void *v_new_c,
                                         const void *v_old, const int32_t *cand_idx, float *dev,
                                         int32_t *sel_local, int32_t *sel_global, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_devtopk(geom, rg, source, k_new_c, k_cached, v_new_c, v_old, cand_idx, dev,
                          sel_local, sel_global));
  const int32_t m = rg->h_cand_off[rg->n_req];
  CB_TRY(hip_status(launch_dev_source(geom, source, k_new_c, k_cached, v_new_c, v_old, cand_idx,
                                      dev, m, (hipStream_t)stream),
                    "deviation"));
  if (rg->h_sel_off[rg->n_req] == 0) return CB_OK;
  return hip_status(cb::launch_topk(rg->n_req, dev, cand_idx, rg->cand_off, rg->sel_off,
                                    sel_local, sel_global, rg->h_cand_off, rg->h_sel_off,
                                    (hipStream_t)stream),
                    "topk");
}

CB_EXPORT cb_status cb_deviation_topk(const cb_geom *geom, const cb_ragged *rg,
                                      const void *v_new_c, const void *v_old,
                                      const int32_t *cand_idx, float *dev, int32_t *sel_local,
                                      int32_t *sel_global, void *stream) {
  return cb_kv_deviation_topk(geom, rg, CB_DEV_V, nullptr, nullptr, v_new_c, v_old, cand_idx,
                              dev, sel_local, sel_global, stream);
}

CB_EXPORT cb_status cb_topk(const cb_ragged *rg, const float *dev, const int32_t *cand_idx,
                            int32_t *sel_local, int32_t *sel_global, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_topk(rg, dev, cand_idx, sel_local, sel_global));
  if (rg->h_sel_off[rg->n_req] == 0) return CB_OK;
  return hip_status(cb::launch_topk(rg->n_req, dev, cand_idx, rg->cand_off, rg->sel_off,
                                    sel_local, sel_global, rg->h_cand_off, rg->h_sel_off,
                                    (hipStream_t)stream),
                    "topk");
}

CB_EXPORT cb_status cb_check_indices(const cb_ragged *rg, const int32_t *cand_idx,
                                     const int32_t *sel_local, const int32_t *sel_global,
                                     int32_t *flags, void *stream) {
  g_last_error.clear();
  if (!flags) return fail(CB_ERR_INVALID_ARG, "flags is NULL");
  const bool cands = cand_idx || sel_local;
  CB_TRY(check_ragged(rg, true, cands, sel_local || sel_global));
  return hip_status(cb::launch_check_indices(rg->tok_off, cands ? rg->cand_off : nullptr,
                                             rg->sel_off, rg->n_req, cand_idx, sel_local,
                                             sel_global, flags, (hipStream_t)stream),
                    "check_indices");
}

CB_EXPORT cb_status cb_fuse_scatter(const cb_geom *geom, void *k_fused, void *v_fused,
                                    const void *k_new_c, const void *v_new_c,
                                    const int32_t *sel_local, const int32_t *sel_global,
                                    int64_t k_total, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_fuse(geom, k_fused, v_fused, k_new_c, v_new_c, sel_local, sel_global, k_total));
  if (k_total == 0) return CB_OK;
  return hip_status(cb::launch_fuse(k_fused, v_fused, k_new_c, v_new_c, sel_local, sel_global,
                                    k_total, (int32_t)(row_elems(geom) * elem_size(geom->dtype)),
                                    nullptr, 0, (hipStream_t)stream),
                    "fuse_scatter");
}

CB_EXPORT cb_status cb_rerotate_fuse(const cb_geom *geom, void *k, void *v, const void *k_new_c,
                                     const void *v_new_c, const int32_t *delta,
                                     const int32_t *sel_local, const int32_t *sel_global,
                                     int64_t k_total, int64_t n_tok, double rope_theta,
                                     int32_t rope_style, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_rerotate(geom, k, k, delta, n_tok, 1, rope_theta, rope_style));
  CB_TRY(validate_fuse(geom, k, v, k_new_c, v_new_c, sel_local, sel_global, k_total));
  CB_TRY(need_ptr(v, "v", n_tok > 0));
  if (k_total > n_tok)
    return fail(CB_ERR_INVALID_ARG, "k_total %lld exceeds n_tok %lld", (long long)k_total,
                (long long)n_tok);
  if (n_tok == 0) return CB_OK;
  return hip_status(cb::launch_rerotate_fuse(geom->dtype, rope_style, k, v, k_new_c, v_new_c,
                                             delta, sel_local, sel_global, k_total, n_tok,
                                             geom->n_kv_heads, geom->head_dim,
                                             rope_table(geom->head_dim, rope_theta), nullptr, 0,
                                             (hipStream_t)stream),
                    "rerotate_fuse");
}

CB_EXPORT cb_status cb_partial_attn(const cb_geom *geom, const cb_ragged *rg, void *out,
                                    const void *q_c, const int32_t *sel_local,
                                    const int32_t *sel_global, const void *k_fused,
                                    const void *v_fused, float softmax_scale, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  CB_TRY(validate_attn(geom, rg, out, q_c, sel_local, sel_global, k_fused, v_fused,
                       softmax_scale));
  CB_TRY(need_ptr(workspace, "workspace", workspace_bytes > 0));
  const cb::AttnPlan plan = plan_attn(geom, rg, workspace ? workspace_bytes : 0);
  return run_attn(geom, rg, plan, out, q_c, sel_local, sel_global, k_fused, v_fused,
                  softmax_scale, workspace, false, (hipStream_t)stream);
}

CB_EXPORT cb_status cb_partial_attn_with_plan(const cb_geom *geom, const cb_ragged *rg,
                                              const cb_attn_plan *plan, void *out,
                                              const void *q_c, const int32_t *sel_local,
                                              const int32_t *sel_global, const void *k_fused,
                                              const void *v_fused, float softmax_scale,
                                              void *workspace, size_t workspace_bytes,
                                              uint32_t flags, void *stream) {
  g_last_error.clear();
  if (!plan) return fail(CB_ERR_INVALID_ARG, "plan is NULL");
  if (flags & ~CB_ATTN_COUNTERS_ZERO)
    return fail(CB_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)flags);
  CB_TRY(validate_attn(geom, rg, out, q_c, sel_local, sel_global, k_fused, v_fused,
                       softmax_scale));
  CB_TRY(need_ptr(workspace, "workspace", workspace_bytes > 0));
  cb::AttnPlan pl;
  CB_TRY(pinned_plan(geom, rg, plan, workspace ? workspace_bytes : 0, pl));
  return run_attn(geom, rg, pl, out, q_c, sel_local, sel_global, k_fused, v_fused,
                  softmax_scale, workspace, (flags & CB_ATTN_COUNTERS_ZERO) != 0,
                  (hipStream_t)stream);
}

CB_EXPORT cb_status cb_partial_attn_workspace_size(const cb_geom *geom, const cb_ragged *rg,
                                                   size_t *bytes) {
  g_last_error.clear();
  if (!bytes) return fail(CB_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  CB_TRY(check_geom(geom));
  CB_TRY(check_ragged(rg, true, false, true));
  *bytes = plan_attn(geom, rg, SIZE_MAX).ws_bytes;
  return CB_OK;
}

namespace {
void export_plan(const cb_geom *geom, const cb_ragged *rg, const cb::AttnPlan &pl,
                 cb_attn_plan *plan) {
  *plan = cb_attn_plan{};
  if (pl.rows_per_tile == 0) {
    plan->workgroups = (int64_t)rg->h_sel_off[rg->n_req] * geom->n_q_heads;
    return;
  }
  plan->mfma = 1;
  plan->key_split = pl.key_split;
  plan->rows_per_tile = pl.rows_per_tile;
  plan->key_chunk = pl.split && pl.spans == 0 ? pl.key_chunk : 0;
  plan->stream_spans = pl.spans;
  plan->tiles = pl.tiles;
  plan->workgroups = pl.units * geom->n_kv_heads;
  plan->workspace_bytes = pl.ws_bytes;
}
}  // namespace

CB_EXPORT cb_status cb_partial_attn_plan(const cb_geom *geom, const cb_ragged *rg,
                                         size_t workspace_bytes, cb_attn_plan *plan) {
  g_last_error.clear();
  if (!plan) return fail(CB_ERR_INVALID_ARG, "plan is NULL");
  *plan = cb_attn_plan{};
  CB_TRY(check_geom(geom));
  CB_TRY(check_ragged(rg, true, false, true));
  export_plan(geom, rg, plan_attn(geom, rg, workspace_bytes), plan);
  return CB_OK;
}

CB_EXPORT cb_status cb_partial_attn_describe_plan(const cb_geom *geom, const cb_ragged *rg,
                                                  cb_attn_plan *plan) {
  g_last_error.clear();
  if (!plan) return fail(CB_ERR_INVALID_ARG, "plan is NULL");
  CB_TRY(check_geom(geom));
  CB_TRY(check_ragged(rg, true, false, true));
  cb::AttnPlan pl;
  CB_TRY(pinned_plan(geom, rg, plan, SIZE_MAX, pl));
  export_plan(geom, rg, pl, plan);
  return CB_OK;
}

namespace {
// The order of cb_blend_layer's steps (see cb_order): select_first is set
// when the V deviation and the top-k run before a rotate-or-replace launch.
// Without a re-rotation both orders are the same three steps (reported as
// rotate first).
cb_status resolve_order(const cb_layer_args *a, int64_t n_tok, bool &select_first) {
  if (a->order < CB_ORDER_AUTO || a->order > CB_ORDER_SELECT_FIRST)
    return fail(CB_ERR_INVALID_ARG, "order %d is not a cb_order", a->order);
  if (a->order == CB_ORDER_SELECT_FIRST && a->dev_source != CB_DEV_V)
    return fail(CB_ERR_INVALID_ARG,
                "CB_ORDER_SELECT_FIRST needs dev_source CB_DEV_V (a key deviation reads the "
                "re-rotated keys)");
  const bool rotate = a->delta && n_tok > 0;
  if (!rotate || a->order == CB_ORDER_ROTATE_FIRST || a->dev_source != CB_DEV_V) {
    select_first = false;
  } else if (a->order == CB_ORDER_SELECT_FIRST) {
    select_first = true;
  } else {
    const cb_geom *g = &a->geom;
    const int64_t cache = n_tok * row_elems(g) * elem_size(g->dtype);
    select_first = cache <= (int64_t)CB_SELECT_FIRST_MAX_BYTES ||
                   !cb::rerotate_deviation_fits(g->dtype, g->n_kv_heads, g->head_dim);
  }
  return CB_OK;
}
}  // namespace

CB_EXPORT cb_status cb_blend_layer_order(const cb_layer_args *a, int32_t *order) {
  g_last_error.clear();
  if (!a) return fail(CB_ERR_INVALID_ARG, "args is NULL");
  if (!order) return fail(CB_ERR_INVALID_ARG, "order is NULL");
  CB_TRY(check_geom(&a->geom));
  CB_TRY(check_ragged(&a->rg, true, false, false));
  bool after = false;
  CB_TRY(resolve_order(a, a->rg.h_tok_off[a->rg.n_req], after));
  *order = after ? CB_ORDER_SELECT_FIRST : CB_ORDER_ROTATE_FIRST;
  return CB_OK;
}

namespace {
// Every check of cb_blend_layer's arguments but the workspace's, before any
// HIP call; `after` receives the step order.
cb_status validate_blend(const cb_layer_args *a, bool &after) {
  if (!a) return fail(CB_ERR_INVALID_ARG, "args is NULL");
  if (a->flags & ~CB_LAYER_WORKSPACE_ZEROED)
    return fail(CB_ERR_INVALID_ARG, "flags 0x%x: only CB_LAYER_WORKSPACE_ZEROED is defined",
                a->flags);
  const cb_geom *geom = &a->geom;
  const cb_ragged *rg = &a->rg;
  CB_TRY(check_ragged(rg, true, true, true));
  const int64_t n_tok = rg->h_tok_off[rg->n_req];
  if (a->delta)
    CB_TRY(validate_rerotate(geom, a->k, a->k, a->delta, n_tok, 1, a->rope_theta, a->rope_style));
  CB_TRY(validate_devtopk(geom, rg, a->dev_source, a->k_new_c, a->k, a->v_new_c, a->v,
                          a->cand_idx, a->dev, a->sel_local, a->sel_global));
  const int32_t k_total = rg->h_sel_off[rg->n_req];
  CB_TRY(validate_fuse(geom, a->k, a->v, a->k_new_c, a->v_new_c, a->sel_local, a->sel_global,
                       k_total));
  CB_TRY(validate_attn(geom, rg, a->out, a->q_c, a->sel_local, a->sel_global, a->k, a->v,
                       a->softmax_scale));
  return resolve_order(a, n_tok, after);
}

// The launches of one validated layer; the attention's split partials and
// arrival counters go to `ws` (ws_bytes; NULL / 0: no split).  sel_cnt: the
// selection's per-request arrival counters, all zero (NULL: the top-k is its
// own launch); used for a V deviation with at most kSelectMaxRequests
// requests.
cb_status launch_blend(const cb_layer_args *a, bool after, void *ws, size_t ws_bytes,
                       unsigned *sel_cnt, hipStream_t s) {
  const cb_geom *geom = &a->geom;
  const cb_ragged *rg = &a->rg;
  const int64_t n_tok = rg->h_tok_off[rg->n_req];
  const int32_t k_total = rg->h_sel_off[rg->n_req];
  const int32_t m = rg->h_cand_off[rg->n_req];
  const bool rotate = a->delta && n_tok > 0;
  const bool fits_shared = cb::rerotate_deviation_fits(geom->dtype, geom->n_kv_heads,
                                                       geom->head_dim);
  // the top-k inside the deviation launch: a V score, counters to count
  // arrivals in, and a re-rotation (if any) that can share the launch
  const bool in_launch = sel_cnt && a->dev_source == CB_DEV_V && m > 0 &&
                         rg->n_req <= cb::kSelectMaxRequests && (after || !rotate || fits_shared);
  // The plan first: it only reads host mirrors, and a plan that would not fit
  // the workspace must stop the call before anything is enqueued.
  const cb::AttnPlan plan = plan_attn(geom, rg, ws ? ws_bytes : 0);
  if (plan.split && plan.ws_bytes > ws_bytes)
    return fail(CB_ERR_UNSUPPORTED, "the attention split needs %zu bytes of workspace, more than "
                "the %zu available", plan.ws_bytes, ws_bytes);
  if (in_launch) {
    // score and select in one launch; rotate first: the re-rotation shares it
    const bool rot_here = rotate && !after;
    CB_TRY(hip_status(cb::launch_deviation_select(
                          geom->dtype, a->rope_style, rot_here ? a->k : nullptr, a->delta, n_tok,
                          geom->n_kv_heads, geom->head_dim,
                          rope_table(geom->head_dim, a->rope_theta), a->v_new_c, a->v,
                          a->cand_idx, a->dev, rg->n_req, rg->cand_off, rg->sel_off,
                          rg->h_cand_off, a->sel_local, a->sel_global, sel_cnt, s),
                      rot_here ? "rerotate+deviation+topk" : "deviation+topk"));
  } else if (after) {
    // the V deviation and the top-k first; the re-rotation joins the fuse
    CB_TRY(hip_status(launch_dev_source(geom, CB_DEV_V, a->k_new_c, a->k, a->v_new_c, a->v,
                                        a->cand_idx, a->dev, m, s),
                      "deviation"));
  } else if (a->dev_source == CB_DEV_V && rotate && fits_shared) {
    // independent K and V work in one launch (a key deviation instead reads
    // the re-rotated keys, so it follows the re-rotation)
    CB_TRY(hip_status(cb::launch_rerotate_deviation(
                          geom->dtype, a->rope_style, a->k, a->delta, n_tok, geom->n_kv_heads,
                          geom->head_dim, rope_table(geom->head_dim, a->rope_theta), a->v_new_c,
                          a->v, a->cand_idx, a->dev, m, s),
                      "rerotate+deviation"));
  } else {
    if (rotate)
      CB_TRY(hip_status(cb::launch_rerotate(geom->dtype, a->rope_style, a->k, a->k, a->delta,
                                            n_tok, 1, geom->n_kv_heads, geom->head_dim,
                                            rope_table(geom->head_dim, a->rope_theta), s),
                        "rerotate"));
    CB_TRY(hip_status(launch_dev_source(geom, a->dev_source, a->k_new_c, a->k, a->v_new_c, a->v,
                                        a->cand_idx, a->dev, m, s),
                      "deviation"));
  }
  if (k_total > 0 && !in_launch)
    CB_TRY(hip_status(cb::launch_topk(rg->n_req, a->dev, a->cand_idx, rg->cand_off, rg->sel_off,
                                      a->sel_local, a->sel_global, rg->h_cand_off,
                                      rg->h_sel_off, s),
                      "topk"));
  // The fuse launch (or the rotate-or-replace launch) also clears the
  // attention's arrival counters.
  const bool clear = k_total > 0 && plan.rows_per_tile > 0 && plan.split;
  uint32_t *const cnt = clear ? (uint32_t *)((char *)ws + plan.cnt_offset) : nullptr;
  const int64_t n_cnt = clear ? plan.n_cnt : 0;
  if (after && rotate) {
    CB_TRY(hip_status(cb::launch_rerotate_fuse(geom->dtype, a->rope_style, a->k, a->v, a->k_new_c,
                                               a->v_new_c, a->delta, a->sel_local, a->sel_global,
                                               k_total, n_tok, geom->n_kv_heads, geom->head_dim,
                                               rope_table(geom->head_dim, a->rope_theta), cnt,
                                               n_cnt, s),
                      "rerotate_fuse"));
  } else if (k_total > 0) {
    CB_TRY(hip_status(
        cb::launch_fuse(a->k, a->v, a->k_new_c, a->v_new_c, a->sel_local, a->sel_global, k_total,
                        (int32_t)(row_elems(geom) * elem_size(geom->dtype)), cnt, n_cnt, s),
        "fuse_scatter"));
  }
  if (k_total == 0) return CB_OK;
  return run_attn(geom, rg, plan, a->out, a->q_c, a->sel_local, a->sel_global, a->k, a->v,
                  a->softmax_scale, ws, clear, s);
}

// The selection counters at the end of a workspace of `bytes` (the region
// CB_SELECT_COUNTER_BYTES long, 256-byte aligned); the bytes before them
// stay for the attention.
unsigned *select_counters(void *ws, size_t &bytes) {
  if (!ws || bytes < CB_SELECT_COUNTER_BYTES + 256) return nullptr;
  const size_t off = (bytes - CB_SELECT_COUNTER_BYTES) & ~(size_t)255;
  bytes = off;
  return reinterpret_cast<unsigned *>(static_cast<char *>(ws) + off);
}
static_assert(CB_SELECT_COUNTER_BYTES / 4 == cb::kSelectMaxRequests,
              "one selection counter per request");
}  // namespace

CB_EXPORT cb_status cb_blend_layer(const cb_layer_args *a, void *stream) {
  g_last_error.clear();
  // Validate every stage before enqueuing any of them.
  bool after = false;
  CB_TRY(validate_blend(a, after));
  CB_TRY(need_ptr(a->workspace, "workspace", a->workspace_bytes > 0));
  void *ws = a->workspace;
  size_t ws_bytes = ws ? a->workspace_bytes : 0;
  unsigned *sel_cnt =
      (a->flags & CB_LAYER_WORKSPACE_ZEROED) ? select_counters(ws, ws_bytes) : nullptr;
  return launch_blend(a, after, ws, ws_bytes, sel_cnt, (hipStream_t)stream);
}

static_assert(CB_NOALLOC_SCRATCH_BYTES == cb::kNoAllocScratchBytes,
              "the header states the static scratch's size");

CB_EXPORT cb_status cb_blend_layer_noalloc(const cb_layer_args *a, void *stream) {
  g_last_error.clear();
  bool after = false;
  CB_TRY(validate_blend(a, after));
  if (a->workspace || a->workspace_bytes)
    return fail(CB_ERR_INVALID_ARG, "cb_blend_layer_noalloc takes no workspace (it uses the "
                "library's static scratch): pass workspace NULL and workspace_bytes 0");
  void *scratch = nullptr;
  CB_TRY(hip_status(cb::noalloc_scratch(&scratch), "static scratch address"));
  // the array starts zero-filled and every call leaves its selection counters at zero
  size_t bytes = cb::kNoAllocScratchBytes;
  unsigned *sel_cnt = select_counters(scratch, bytes);
  return launch_blend(a, after, scratch, bytes, sel_cnt, (hipStream_t)stream);
}

CB_EXPORT const char *cb_status_str(cb_status status) {
  switch (status) {
    case CB_OK: return "CB_OK";
    case CB_ERR_INVALID_ARG: return "CB_ERR_INVALID_ARG";
    case CB_ERR_UNSUPPORTED: return "CB_ERR_UNSUPPORTED";
    case CB_ERR_HIP: return "CB_ERR_HIP";
  }
  return "unknown cb_status";
}

CB_EXPORT const char *cb_last_error(void) { return g_last_error.c_str(); }

CB_EXPORT int32_t cb_abi_version(void) { return CB_ABI_VERSION; }

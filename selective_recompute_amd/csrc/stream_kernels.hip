// Bandwidth-bound kernels of the blend: key re-rotation, V deviation, the
// per-request top-k selection and the row scatter that fuses the caches.
//
// Pages: [Derivations] = "数学推导" (CacheBlend math derivations page);
// [KV-blog] = "rag的kvcache问题".
#include <algorithm>
#include <climits>

#include "cb_device.hpp"
#include "cb_launch.hpp"

namespace cb {

// ---------------------------------------------------------------------------
// Re-rotation, [Derivations, "CacheBlend 中的应用"]: K_rot = R_delta K_old,
// applied to each D/2 coordinate pairs of every KV head with the 2x2 block of
// [Derivations, "RoPE 位置编码的相对位置不变性证明"].
//
// A thread owns one "unit": VP consecutive pairs of one head (VP = 8 for
// bf16, 4 for fp32 so that each half is one 16-byte access).  Its pairs are
// fixed for the whole kernel, so the cos/sin of its VP angles are computed
// only when delta changes between the tokens it visits (a token's delta is
// the start of its chunk) and are reused across all layers.  The angle is
// reduced in double precision to a fraction of a turn in [-1/2, 1/2]; the
// gfx950 v_sin_f32 / v_cos_f32 instructions take their argument in turns.
// ---------------------------------------------------------------------------
struct RotGeom {
  int64_t n_tok;
  int32_t n_layers, head_dim, units_per_head, units_per_row, tok_per_iter, tok_per_block;
};

// cos / sin of a unit's VP pair angles for position delta d: the angle in
// turns, d * rev[i], reduced to [-1/2, 1/2] in double precision.
template <int VP>
__device__ inline void unit_trig(int d, const double *rev, float *cs, float *sn) {
#pragma unroll
  for (int i = 0; i < VP; ++i) {
    const double turns = (double)d * rev[i];
    const float frac = (float)(turns - rint(turns));  // in [-1/2, 1/2]
    sn[i] = __builtin_amdgcn_sinf(frac);
    cs[i] = __builtin_amdgcn_cosf(frac);
  }
}

// One unit of one row (head base pointers src / dst): load its VP pairs,
// turn them by the 2x2 block (when `turn`), store.  dst == src allowed.
template <typename T, int STYLE>
__device__ inline void rotate_unit(T *dst, const T *src, int j0, int hd, const float *cs,
                                   const float *sn, bool turn) {
  constexpr int VP = Vec16<T>::N;
  float a[VP], b[VP];
  if (STYLE == 0) {  // pairs (j, j + D/2)
    Vec16<T>::load(src + j0, a);
    Vec16<T>::load(src + hd / 2 + j0, b);
  } else {           // pairs (2j, 2j + 1)
    float x0[VP], x1[VP];
    Vec16<T>::load(src + 2 * j0, x0);
    Vec16<T>::load(src + 2 * j0 + VP, x1);
#pragma unroll
    for (int i = 0; i < VP / 2; ++i) {
      a[i] = x0[2 * i]; b[i] = x0[2 * i + 1];
      a[VP / 2 + i] = x1[2 * i]; b[VP / 2 + i] = x1[2 * i + 1];
    }
  }
  if (turn) {
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const float x = a[i], y = b[i];
      a[i] = fmaf(x, cs[i], -y * sn[i]);
      b[i] = fmaf(x, sn[i], y * cs[i]);
    }
  }
  if (STYLE == 0) {
    Vec16<T>::store(dst + j0, a);
    Vec16<T>::store(dst + hd / 2 + j0, b);
  } else {
    float x0[VP], x1[VP];
#pragma unroll
    for (int i = 0; i < VP / 2; ++i) {
      x0[2 * i] = a[i]; x0[2 * i + 1] = b[i];
      x1[2 * i] = a[VP / 2 + i]; x1[2 * i + 1] = b[VP / 2 + i];
    }
    Vec16<T>::store(dst + 2 * j0, x0);
    Vec16<T>::store(dst + 2 * j0 + VP, x1);
  }
}

// Element offsets, inside a head, of a unit's two 16-byte pieces.
template <typename T, int STYLE>
__device__ inline void unit_pieces(int j0, int hd, int &p0, int &p1) {
  constexpr int VP = Vec16<T>::N;
  p0 = STYLE == 0 ? j0 : 2 * j0;
  p1 = STYLE == 0 ? hd / 2 + j0 : 2 * j0 + VP;
}

// tid: the thread's index among the block's units_per_row * tok_per_iter threads.
template <typename T, int STYLE>
__device__ inline void rerotate_block(T *__restrict__ k_out, const T *__restrict__ k_in,
                                      const int32_t *__restrict__ delta, const RotGeom &gm,
                                      const RopeTable &tab, int64_t block, int tid) {
  constexpr int VP = Vec16<T>::N;  // pairs per unit
  if (tid >= gm.units_per_row * gm.tok_per_iter) return;
  const int unit = tid % gm.units_per_row;
  const int slot = tid / gm.units_per_row;
  const int head = unit / gm.units_per_head;
  const int j0 = (unit % gm.units_per_head) * VP;
  const int hd = gm.head_dim;
  const int64_t row_elems = (int64_t)(gm.units_per_row / gm.units_per_head) * hd;
  const bool in_place = (k_out == k_in);

  double rev[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) rev[i] = tab.rev_per_pos[j0 + i];
  float cs[VP], sn[VP];
  int cur = INT_MIN;

  const int64_t t_begin = (int64_t)block * gm.tok_per_block;
  const int64_t t_end = t_begin + gm.tok_per_block < gm.n_tok ? t_begin + gm.tok_per_block : gm.n_tok;
  for (int64_t t = t_begin + slot; t < t_end; t += gm.tok_per_iter) {
    const int d = delta[t];
    if (d == 0 && in_place) continue;  // R_0 = I
    if (d != cur && d != 0) {
      cur = d;
      unit_trig<VP>(d, rev, cs, sn);
    }
    for (int l = 0; l < gm.n_layers; ++l) {
      const int64_t off = ((int64_t)l * gm.n_tok + t) * row_elems + (int64_t)head * hd;
      rotate_unit<T, STYLE>(k_out + off, k_in + off, j0, hd, cs, sn, d != 0);
    }
  }
}

template <typename T>
static RotGeom rot_geom(int64_t n_tok, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                        int64_t &blocks) {
  constexpr int VP = Vec16<T>::N;
  RotGeom gm;
  gm.n_tok = n_tok;
  gm.n_layers = n_layers;
  gm.head_dim = head_dim;
  gm.units_per_head = (head_dim / 2) / VP;
  gm.units_per_row = gm.units_per_head * n_kv_heads;
  gm.tok_per_iter = gm.units_per_row >= 256 ? 1 : 256 / gm.units_per_row;
  // Enough blocks to fill the chip; each block then walks a short contiguous
  // token range so the cached trig is reused within a chunk.
  int64_t iters = (n_tok + (int64_t)gm.tok_per_iter * 2048 - 1) / ((int64_t)gm.tok_per_iter * 2048);
  if (iters < 1) iters = 1;
  if (iters > 16) iters = 16;
  gm.tok_per_block = (int)(gm.tok_per_iter * iters);
  blocks = (n_tok + gm.tok_per_block - 1) / gm.tok_per_block;
  return gm;
}

template <typename T, int STYLE>
__global__ __launch_bounds__(1024) void rerotate_kernel(T *__restrict__ k_out,
                                                        const T *__restrict__ k_in,
                                                        const int32_t *__restrict__ delta,
                                                        RotGeom gm, RopeTable tab) {
  rerotate_block<T, STYLE>(k_out, k_in, delta, gm, tab, blockIdx.x, threadIdx.x);
}

template <typename T, int STYLE>
static hipError_t rerotate_typed(void *k_out, const void *k_in, const int32_t *delta,
                                 int64_t n_tok, int32_t n_layers, int32_t n_kv_heads,
                                 int32_t head_dim, const RopeTable &tab, hipStream_t stream) {
  int64_t blocks;
  const RotGeom gm = rot_geom<T>(n_tok, n_layers, n_kv_heads, head_dim, blocks);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rerotate_kernel<T, STYLE>), dim3((unsigned)blocks),
                     dim3(gm.units_per_row * gm.tok_per_iter), 0, stream, (T *)k_out,
                     (const T *)k_in, delta, gm, tab);
  return hipGetLastError();
}

hipError_t launch_rerotate(int dtype, int style, void *k_out, const void *k_in,
                           const int32_t *delta, int64_t n_tok, int32_t n_layers,
                           int32_t n_kv_heads, int32_t head_dim, const RopeTable &tab,
                           hipStream_t stream) {
  if (dtype == kBF16)
    return style == 0 ? rerotate_typed<bf16, 0>(k_out, k_in, delta, n_tok, n_layers, n_kv_heads, head_dim, tab, stream)
                      : rerotate_typed<bf16, 1>(k_out, k_in, delta, n_tok, n_layers, n_kv_heads, head_dim, tab, stream);
  return style == 0 ? rerotate_typed<float, 0>(k_out, k_in, delta, n_tok, n_layers, n_kv_heads, head_dim, tab, stream)
                    : rerotate_typed<float, 1>(k_out, k_in, delta, n_tok, n_layers, n_kv_heads, head_dim, tab, stream);
}

// ---------------------------------------------------------------------------
// Deviation, [Derivations, "近似解"]: dev[j] = ||V_new_c[j] - V_old[cand[j]]||^2
// over all KV heads and dims.  [KV-blog, "核心发现： KV 偏差"] measures the
// token's whole KV vector: with NT = 2 the wave adds the squared distance of a
// second pair of tensors (K, the cached keys already at the new position) to
// the same sum.  One wave per candidate row, 16-byte loads, fp32 fused
// multiply-add accumulation, butterfly reduction across the wave.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float sq_dist_share(const T *__restrict__ a, const T *__restrict__ b, int lane,
                                      int nvec, float acc) {
  constexpr int V = Vec16<T>::N;
  for (int v = lane; v < nvec; v += kWave) {
    float x[V], y[V];
    Vec16<T>::load(a + v * V, x);
    Vec16<T>::load(b + v * V, y);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float df = x[i] - y[i];
      acc = fmaf(df, df, acc);
    }
  }
  return acc;
}

template <typename T, int NT>
__device__ inline void deviation_block(const T *__restrict__ new0, const T *__restrict__ old0,
                                       const T *__restrict__ new1, const T *__restrict__ old1,
                                       const int32_t *__restrict__ cand_idx,
                                       float *__restrict__ dev, int64_t m, int32_t row_elems,
                                       int64_t block, int64_t n_blocks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (block * blockDim.x + threadIdx.x) / kWave;
  const int64_t n_waves = (n_blocks * blockDim.x) / kWave;
  const int nvec = row_elems / Vec16<T>::N;
  for (int64_t j = wave; j < m; j += n_waves) {
    const int64_t c = cand_idx[j];
    float acc = sq_dist_share(new0 + j * row_elems, old0 + c * row_elems, lane, nvec, 0.f);
    if (NT == 2) acc = sq_dist_share(new1 + j * row_elems, old1 + c * row_elems, lane, nvec, acc);
    acc = wave_sum(acc);
    if (lane == 0) dev[j] = acc;
  }
}

template <typename T, int NT>
__global__ __launch_bounds__(256) void deviation_kernel(
    const T *__restrict__ new0, const T *__restrict__ old0, const T *__restrict__ new1,
    const T *__restrict__ old1, const int32_t *__restrict__ cand_idx, float *__restrict__ dev,
    int64_t m, int32_t row_elems) {
  deviation_block<T, NT>(new0, old0, new1, old1, cand_idx, dev, m, row_elems, blockIdx.x,
                         gridDim.x);
}

static int64_t deviation_blocks(int64_t m) {
  int64_t blocks = (m + 3) / 4;  // 4 waves per block, one row per wave
  return blocks > 8192 ? 8192 : blocks;
}

template <typename T>
static void deviation_typed(const void *new0, const void *old0, const void *new1,
                            const void *old1, const int32_t *cand_idx, float *dev, int64_t m,
                            int32_t row_elems, hipStream_t stream) {
  const dim3 grid((unsigned)deviation_blocks(m)), block(256);
  if (new1)
    hipLaunchKernelGGL((deviation_kernel<T, 2>), grid, block, 0, stream, (const T *)new0,
                       (const T *)old0, (const T *)new1, (const T *)old1, cand_idx, dev, m,
                       row_elems);
  else
    hipLaunchKernelGGL((deviation_kernel<T, 1>), grid, block, 0, stream, (const T *)new0,
                       (const T *)old0, (const T *)nullptr, (const T *)nullptr, cand_idx, dev, m,
                       row_elems);
}

hipError_t launch_deviation(int dtype, const void *new0, const void *old0, const void *new1,
                            const void *old1, const int32_t *cand_idx, float *dev, int64_t m,
                            int32_t row_elems, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  if (dtype == kBF16)
    deviation_typed<bf16>(new0, old0, new1, old1, cand_idx, dev, m, row_elems, stream);
  else
    deviation_typed<float>(new0, old0, new1, old1, cand_idx, dev, m, row_elems, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-rotation of K and deviation of V in one launch: the two are independent
// (they touch different tensors), and at small sizes neither fills the chip
// alone.  Blocks [0, rot_blocks) re-rotate, the rest score candidates.
// ---------------------------------------------------------------------------
template <typename T, int STYLE>
__global__ __launch_bounds__(256) void rerotate_deviation_kernel(
    T *__restrict__ k, const int32_t *__restrict__ delta, RotGeom gm, RopeTable tab,
    int64_t rot_blocks, const T *__restrict__ v_new_c, const T *__restrict__ v_old,
    const int32_t *__restrict__ cand_idx, float *__restrict__ dev, int64_t m, int32_t row_elems) {
  if ((int64_t)blockIdx.x < rot_blocks)
    rerotate_block<T, STYLE>(k, k, delta, gm, tab, blockIdx.x, threadIdx.x);
  else
    deviation_block<T, 1>(v_new_c, v_old, nullptr, nullptr, cand_idx, dev, m, row_elems,
                          blockIdx.x - rot_blocks, gridDim.x - rot_blocks);
}

template <typename T, int STYLE>
static hipError_t rerotate_deviation_typed(void *k, const int32_t *delta, int64_t n_tok,
                                           int32_t n_kv_heads, int32_t head_dim,
                                           const RopeTable &tab, const void *v_new_c,
                                           const void *v_old, const int32_t *cand_idx,
                                           float *dev, int64_t m, hipStream_t stream) {
  int64_t rot_blocks;
  const RotGeom gm = rot_geom<T>(n_tok, 1, n_kv_heads, head_dim, rot_blocks);
  const int64_t dev_blocks = m > 0 ? deviation_blocks(m) : 0;
  if (rot_blocks + dev_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rerotate_deviation_kernel<T, STYLE>), dim3((unsigned)(rot_blocks + dev_blocks)),
                     dim3(256), 0, stream, (T *)k, delta, gm, tab, rot_blocks,
                     (const T *)v_new_c, (const T *)v_old, cand_idx, dev, m,
                     (int32_t)(n_kv_heads * head_dim));
  return hipGetLastError();
}

bool rerotate_deviation_fits(int dtype, int32_t n_kv_heads, int32_t head_dim) {
  const int vp = dtype == kBF16 ? 8 : 4;
  return (head_dim / 2) / vp * n_kv_heads <= 256;  // one re-rotation row per 256 threads
}

hipError_t launch_rerotate_deviation(int dtype, int style, void *k, const int32_t *delta,
                                     int64_t n_tok, int32_t n_kv_heads, int32_t head_dim,
                                     const RopeTable &tab, const void *v_new_c,
                                     const void *v_old, const int32_t *cand_idx, float *dev,
                                     int64_t m, hipStream_t stream) {
#define CB_RD(T, S) \
  rerotate_deviation_typed<T, S>(k, delta, n_tok, n_kv_heads, head_dim, tab, v_new_c, v_old, cand_idx, dev, m, stream)
  if (dtype == kBF16) return style == 0 ? CB_RD(bf16, 0) : CB_RD(bf16, 1);
  return style == 0 ? CB_RD(float, 0) : CB_RD(float, 1);
#undef CB_RD
}

// ---------------------------------------------------------------------------
// Top-k, [Derivations, "近似解"] (greedy TopK of the deviation) with ties to
// the lower index and NaN above +inf.  One 1024-thread workgroup per request.
// Wave w owns the contiguous candidate range [w cw, (w + 1) cw) of its
// request (cw = ceil(m / 16) rounded up to 64), and in round i its lane l holds
// candidate w cw + 64 i + l: every load is one coalesced 256-byte run, and the
// scores stay in registers for up to KPT rounds (KPT = 0: re-read every pass).
//   1. MSB-first radix select over the order-preserving uint32 key of each
//      fp32 score, 8 bits per pass with an LDS histogram (a wave counts its
//      first two distinct bins in registers over all its rounds and adds them
//      once per pass; other bins one atomic per lane).  The select
//      stops at the first
//      pass whose boundary bin holds exactly the keys still missing: then the
//      whole bin is selected.
//   2. An ordered compaction emits, in candidate order (= ascending packed
//      row), every key above the boundary bin and the first `keep_eq` keys
//      inside it (ties to the lower index): one scan over the 16 waves' counts
//      gives each wave's bases, and inside a round the ballot of the same
//      predicate orders the lanes (its bits below the lane).
// ---------------------------------------------------------------------------
__device__ inline uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0xFFFFFFFFu;          // NaN ranks first
  if (u == 0x80000000u) u = 0u;            // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

// Rounds of 64 candidates per wave for a request of m candidates.
__host__ __device__ constexpr int topk_rounds(int m) {
  return ((m + kTopkWaves - 1) / kTopkWaves + kWave - 1) / kWave;
}

// Inclusive prefix sum over the 64 lanes of a wave, lane 0 first: shifted
// adds inside each row of 16 lanes (DPP row_shr 1, 2, 4, 8, lanes shifted
// in from outside the row reading 0), then the last lane of row 0 added to
// row 1 and of row 2 to row 3 (row_bcast:15), then lane 31 to rows 2 and 3
// (row_bcast:31) -- gfx9's cross-lane data paths, no LDS round trips.
__device__ inline uint32_t wave_prefix_sum(uint32_t x) {
  const int v = (int)x;
  int s = v;
  s += __builtin_amdgcn_update_dpp(0, s, 0x111, 0xf, 0xf, true);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xf, 0xf, true);  // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xf, 0xf, true);  // row_shr:4
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xf, 0xf, true);  // row_shr:8
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return (uint32_t)s;
}

// A wave's contribution to the LDS histogram of one radix pass.  Most scores
// share their leading bits (the deviation tiers), so a wave's keys fall into
// very few bins: the first two distinct bins it meets are counted in
// registers over all of its rounds and added with one atomic each when the
// pass ends (flush); keys in any other bin add one atomic per lane.  Atomics
// of 16 waves on the same one or two LDS words, one per wave and round,
// serialised the pass before (26.6k of the 66k cycles at 32k candidates).
struct WaveHist {
  int bin[2] = {-1, -1};
  uint32_t cnt[2] = {0u, 0u};

  __device__ void add(uint32_t *hist, int b) {
    const int lane = (int)(threadIdx.x & (kWave - 1));
    uint64_t pending = __ballot(b >= 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!pending) return;
      if (bin[j] < 0) {  // first use of this slot: the lowest pending lane's bin
        bin[j] = __builtin_amdgcn_readlane(b, __builtin_ctzll(pending));
      }
      const uint64_t same = __ballot(b == bin[j]);
      cnt[j] += (uint32_t)__popcll(same);
      pending &= ~same;
    }
    if ((pending >> lane) & 1ull) atomicAdd(&hist[b], 1u);
  }
  __device__ void flush(uint32_t *hist) const {
    if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (bin[j] >= 0 && cnt[j]) atomicAdd(&hist[bin[j]], cnt[j]);
    }
  }
};

// Shared memory of one workgroup's top-k.
struct TopkShared {
  uint32_t hist[256];
  uint32_t digit, above, count;
  uint32_t wave_tot[2][kTopkWaves];
};

// Selects k of the m scores dev[c0 .. c0 + m) of one request (candidates
// cand_idx[c0 ..]) into sel_local / sel_global [s0 .. s0 + k), ascending,
// with the whole 1024-thread workgroup.  AGENT: the scores were written by
// other workgroups of the same launch and are read at agent scope.  May be
// called again by the same workgroup for another request.
template <int KPT, bool AGENT>
__device__ __attribute__((always_inline)) void topk_select(TopkShared &sh, const float *__restrict__ dev,
                            const int32_t *__restrict__ cand_idx, int c0, int m, int s0, int k,
                            int32_t *__restrict__ sel_local, int32_t *__restrict__ sel_global) {
  __syncthreads();  // a previous call's readers of sh are done
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (k <= 0) return;
  if (k >= m) {  // every candidate is selected
    for (int j = tid; j < m; j += kTopkThreads) {
      sel_local[s0 + j] = c0 + j;
      sel_global[s0 + j] = cand_idx[c0 + j];
    }
    return;
  }
  if (tid < 256) sh.hist[tid] = 0;  // the first pass's histogram, cleared while the scores load
  const int rounds = topk_rounds(m);
  const int wb = wave * rounds * kWave;                  // first candidate of this wave
  const int n_w = max(0, min(m - wb, rounds * kWave));   // candidates of this wave
  const float *dw = dev + c0 + wb + lane;
  auto score = [&](int off) -> float {  // scores another workgroup may have written: agent scope
    return AGENT ? __uint_as_float(load_agent(reinterpret_cast<const uint32_t *>(dw + off)))
                 : dw[off];
  };
  const int32_t *cw = cand_idx + c0 + wb + lane;
  uint32_t keys[KPT > 0 ? KPT : 1];
  int32_t cands[KPT > 0 ? KPT : 1];  // loaded with the scores: no load left at the end
  if (KPT > 0) {
#pragma unroll
    for (int i = 0; i < (KPT > 0 ? KPT : 1); ++i) {
      const bool ok = kWave * i + lane < n_w;
      keys[i] = ok ? order_key(score(kWave * i)) : 0u;
      cands[i] = ok ? cw[kWave * i] : 0;
    }
  }
  auto key_at = [&](int i) -> uint32_t {  // only for candidates of this wave
    if (KPT > 0) return keys[i];
    return order_key(score(kWave * i));
  };
  const int iters = KPT > 0 ? KPT : rounds;  // uniform over the workgroup
  constexpr int kUnroll = KPT > 0 ? KPT : 1;  // register path: fully unrolled

  uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (pass > 0 && tid < 256) sh.hist[tid] = 0;
    // The zeros are visible, and every thread has read the previous pass's
    // sh_*; the first pass's score loads may still be in flight.
    phase_barrier();
    WaveHist wh;
#pragma unroll kUnroll
    for (int i = 0; i < iters; ++i) {
      int bin = -1;
      if (kWave * i + lane < n_w) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) bin = (int)((key >> shift) & 255u);
      }
      wh.add(sh.hist, bin);
    }
    wh.flush(sh.hist);
    __syncthreads();
    if (tid < kWave) {
      // Lane l holds bins 255 - 4l down to 252 - 4l, so a prefix sum over
      // the lanes counts every key in this lane's bins and the bins above.
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = sh.hist[255 - 4 * tid - q];
      const uint32_t tot = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_prefix_sum(tot);
      uint32_t above = incl - tot;
      if (above < krem && incl >= krem) {
        for (int q = 0; q < 4; ++q) {
          if (above + h[q] >= krem) {
            sh.digit = 255 - 4 * tid - q; sh.above = above; sh.count = h[q];
            break;
          }
          above += h[q];
        }
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    krem -= sh.above;
    if (sh.count == krem) break;  // the whole boundary bin is selected
  }
  const uint32_t keep_eq = krem;  // keys of the boundary bin to keep, lowest index first

  // keys above the boundary bin (gt) and inside it (eq), per wave
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll kUnroll
  for (int i = 0; i < iters; ++i) {
    bool gt = false, eq = false;
    if (kWave * i + lane < n_w) {
      const uint32_t km = key_at(i) & mask;
      gt = km > prefix;
      eq = km == prefix;
    }
    n_gt += __popcll(__ballot(gt));
    n_eq += __popcll(__ballot(eq));
  }
  if (lane == 0) {
    sh.wave_tot[0][wave] = n_gt;
    sh.wave_tot[1][wave] = n_eq;
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;  // of the waves before this one
  for (int w = 0; w < wave; ++w) {
    gt_before += sh.wave_tot[0][w];
    eq_before += sh.wave_tot[1][w];
  }
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
#pragma unroll kUnroll
  for (int i = 0; i < iters; ++i) {
    bool gt = false, eq = false;
    if (kWave * i + lane < n_w) {
      const uint32_t km = key_at(i) & mask;
      gt = km > prefix;
      eq = km == prefix;
    }
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const uint32_t g_pos = gt_before + (uint32_t)__popcll(bg & below);
    const uint32_t e_pos = eq_before + (uint32_t)__popcll(be & below);
    const uint32_t pos = g_pos + (e_pos < keep_eq ? e_pos : keep_eq);
    if ((gt || (eq && e_pos < keep_eq)) && pos < (uint32_t)k) {  // pos < k always: a guard
      sel_local[s0 + pos] = c0 + wb + kWave * i + lane;
      sel_global[s0 + pos] = KPT > 0 ? cands[i] : cw[kWave * i];
    }
    gt_before += (uint32_t)__popcll(bg);
    eq_before += (uint32_t)__popcll(be);
  }
}

// one_m / one_k: for a single request, its candidate and selected counts
// (known on the host), so the scores are loaded without first waiting for
// the offsets; -1 with several requests.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *__restrict__ dev, const int32_t *__restrict__ cand_idx,
    const int32_t *__restrict__ cand_off, const int32_t *__restrict__ sel_off,
    int32_t *__restrict__ sel_local, int32_t *__restrict__ sel_global, int32_t one_m,
    int32_t one_k) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const bool one = one_m >= 0;
  const int c0 = one ? 0 : cand_off[r];
  const int m = one ? one_m : cand_off[r + 1] - c0;
  const int s0 = one ? 0 : sel_off[r];
  const int k = one ? one_k : sel_off[r + 1] - s0;
  topk_select<KPT, false>(sh, dev, cand_idx, c0, m, s0, k, sel_local, sel_global);
}

hipError_t launch_topk(int32_t n_req, const float *dev, const int32_t *cand_idx,
                       const int32_t *cand_off, const int32_t *sel_off, int32_t *sel_local,
                       int32_t *sel_global, const int32_t *h_cand_off, const int32_t *h_sel_off,
                       hipStream_t stream) {
  if (n_req == 0) return hipSuccess;
  int32_t max_m = 0;
  for (int32_t r = 0; r < n_req; ++r) max_m = std::max(max_m, h_cand_off[r + 1] - h_cand_off[r]);
  const int32_t one_m = n_req == 1 ? h_cand_off[1] : -1;
  const int32_t one_k = n_req == 1 ? h_sel_off[1] : -1;
  const int rounds = topk_rounds(max_m);
#define CB_TOPK(K)                                                                            \
  hipLaunchKernelGGL(topk_kernel<K>, dim3(n_req), dim3(kTopkThreads), 0, stream, dev, cand_idx, \
                     cand_off, sel_off, sel_local, sel_global, one_m, one_k)
  if (rounds <= 1) CB_TOPK(1);
  else if (rounds <= 2) CB_TOPK(2);
  else if (rounds <= 4) CB_TOPK(4);
  else if (rounds <= 8) CB_TOPK(8);
  else if (rounds <= 16) CB_TOPK(16);
  else if (rounds <= 32) CB_TOPK(32);
  else CB_TOPK(0);
#undef CB_TOPK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// V deviation and top-k in one launch (cb_blend_layer on a workspace that
// started zero-filled).  Workgroup b scores candidates [16 b, 16 b + 16), one
// wave per row ([Derivations, "近似解"] score, as deviation_kernel), and
// stores each score at agent scope.  Once those stores have completed it
// adds 1 to the arrival counter of every request its rows belong to; the
// workgroup that completes a request's count sets the counter back to zero
// and selects that request's rows itself (topk_select), so the selection
// needs no launch of its own and every launch leaves its counters at zero.
// ROT: the same launch re-rotates K in place ([Derivations, "CacheBlend 中的
// 应用"]) in the workgroups after the scoring ones, four 256-thread
// re-rotation blocks each; the selections then run while the longer
// re-rotation still streams.
// ---------------------------------------------------------------------------
constexpr int kSelRows = kTopkWaves;  // candidates scored per workgroup

template <typename T, int KPT, int ROT, int STYLE>
__global__ __launch_bounds__(kTopkThreads) void deviation_select_kernel(
    const T *__restrict__ v_new_c, const T *__restrict__ v_old,
    const int32_t *__restrict__ cand_idx, float *__restrict__ dev, int64_t m, int32_t row_elems,
    const int32_t *__restrict__ cand_off, const int32_t *__restrict__ sel_off, int32_t n_req,
    int32_t *__restrict__ sel_local, int32_t *__restrict__ sel_global, unsigned *__restrict__ cnt,
    int64_t dev_blocks, T *__restrict__ k, const int32_t *__restrict__ delta, RotGeom gm,
    RopeTable tab, int64_t rot_blocks) {
  if (ROT && (int64_t)blockIdx.x >= dev_blocks) {  // uniform
    const int64_t rb = ((int64_t)blockIdx.x - dev_blocks) * 4 + threadIdx.x / 256;
    if (rb < rot_blocks) rerotate_block<T, STYLE>(k, k, delta, gm, tab, rb, threadIdx.x & 255);
    return;
  }
  __shared__ TopkShared sh;
  __shared__ int s_req[kSelRows];  // requests this workgroup completes (at most one per row)
  __shared__ int s_n;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t j0 = (int64_t)blockIdx.x * kSelRows;
  const int64_t j1 = j0 + kSelRows < m ? j0 + kSelRows : m;
  const int64_t j = j0 + wave;
  if (j < m) {
    const int64_t c = cand_idx[j];
    float acc = sq_dist_share(v_new_c + j * row_elems, v_old + c * row_elems, lane,
                              row_elems / Vec16<T>::N, 0.f);
    acc = wave_sum(acc);
    if (lane == 0) store_agent(reinterpret_cast<uint32_t *>(dev + j), __float_as_uint(acc));
  }
  if (threadIdx.x == 0) s_n = 0;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's score has reached the coherence point
  __syncthreads();
  for (int r = threadIdx.x; r < n_req; r += kTopkThreads) {
    const int c0 = cand_off[r], c1 = cand_off[r + 1];
    if (c1 > c0 && c0 < j1 && c1 > j0) {
      const unsigned need = (unsigned)((c1 - 1) / kSelRows - c0 / kSelRows + 1);
      const unsigned prev =
          __hip_atomic_fetch_add(cnt + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == need - 1) {
        store_agent(cnt + r, 0u);
        s_req[atomicAdd(&s_n, 1)] = r;
      }
    }
  }
  __syncthreads();
  const int n_done = s_n;
  for (int i = 0; i < n_done; ++i) {
    const int r = s_req[i];
    const int c0 = cand_off[r], s0 = sel_off[r];
    topk_select<KPT, true>(sh, dev, cand_idx, c0, cand_off[r + 1] - c0, s0, sel_off[r + 1] - s0,
                           sel_local, sel_global);
  }
}

template <typename T, int KPT>
static void deviation_select_typed(int style, void *k, const int32_t *delta, int64_t n_tok,
                                   int32_t n_kv_heads, int32_t head_dim, const RopeTable &tab,
                                   const void *v_new_c, const void *v_old,
                                   const int32_t *cand_idx, float *dev, int64_t m,
                                   int32_t n_req, const int32_t *cand_off,
                                   const int32_t *sel_off, int32_t *sel_local,
                                   int32_t *sel_global, unsigned *cnt, hipStream_t stream) {
  const int64_t dev_blocks = (m + kSelRows - 1) / kSelRows;
  const int32_t row_elems = n_kv_heads * head_dim;
  int64_t rot_blocks = 0;
  RotGeom gm{};
  if (k) gm = rot_geom<T>(n_tok, 1, n_kv_heads, head_dim, rot_blocks);
  const int64_t blocks = dev_blocks + (rot_blocks + 3) / 4;
  if (blocks == 0) return;
#define CB_DS(R, S)                                                                                \
  hipLaunchKernelGGL((deviation_select_kernel<T, KPT, R, S>), dim3((unsigned)blocks),                \
                     dim3(kTopkThreads), 0, stream, (const T *)v_new_c, (const T *)v_old, cand_idx, \
                     dev, m, row_elems, cand_off, sel_off, n_req, sel_local, sel_global, cnt,     \
                     dev_blocks, (T *)k, delta, gm, tab, rot_blocks)
  if (!k) CB_DS(0, 0);
  else if (style == 0) CB_DS(1, 0);
  else CB_DS(1, 1);
#undef CB_DS
}

hipError_t launch_deviation_select(int dtype, int style, void *k, const int32_t *delta,
                                   int64_t n_tok, int32_t n_kv_heads, int32_t head_dim,
                                   const RopeTable &tab, const void *v_new_c, const void *v_old,
                                   const int32_t *cand_idx, float *dev, int32_t n_req,
                                   const int32_t *cand_off, const int32_t *sel_off,
                                   const int32_t *h_cand_off, int32_t *sel_local,
                                   int32_t *sel_global, unsigned *cnt, hipStream_t stream) {
  int32_t max_m = 0;
  for (int32_t r = 0; r < n_req; ++r) max_m = std::max(max_m, h_cand_off[r + 1] - h_cand_off[r]);
  const int64_t m = h_cand_off[n_req];
  const int rounds = topk_rounds(max_m);
#define CB_DSEL(K)                                                                            \
  deviation_select_typed<T, K>(style, k, delta, n_tok, n_kv_heads, head_dim, tab, v_new_c,   \
                               v_old, cand_idx, dev, m, n_req, cand_off, sel_off, sel_local, \
                               sel_global, cnt, stream)
  auto run = [&](auto tag) {
    using T = decltype(tag);
    if (rounds <= 2) CB_DSEL(2);
    else if (rounds <= 8) CB_DSEL(8);
    else if (rounds <= 32) CB_DSEL(32);
    else CB_DSEL(0);
  };
#undef CB_DSEL
  if (dtype == kBF16) run(bf16{});
  else run(float{});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Index preconditions, checked on the device (cb_check_indices): one
// 1024-thread workgroup walks every request's candidates and selections and
// ORs the violations it finds; the workgroup's OR is written to *flags, so
// the word needs no clearing beforehand.  Reads only the arrays it is given.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void check_indices_kernel(
    const int32_t *__restrict__ tok_off, const int32_t *__restrict__ cand_off,
    const int32_t *__restrict__ sel_off, int32_t n_req, const int32_t *__restrict__ cand_idx,
    const int32_t *__restrict__ sel_local, const int32_t *__restrict__ sel_global,
    int32_t *__restrict__ flags) {
  __shared__ int32_t s_flags;
  if (threadIdx.x == 0) s_flags = 0;
  __syncthreads();
  int32_t f = 0;
  for (int32_t r = 0; r < n_req; ++r) {
    const int32_t t0 = tok_off[r], t1 = tok_off[r + 1];
    if (cand_idx) {
      const int32_t c0 = cand_off[r], c1 = cand_off[r + 1];
      for (int32_t j = c0 + (int32_t)threadIdx.x; j < c1; j += kTopkThreads) {
        const int32_t c = cand_idx[j];
        if (c < t0 || c >= t1) f |= 1;                       // CB_CHECK_CAND_RANGE
        if (j > c0 && cand_idx[j - 1] >= c) f |= 2;          // CB_CHECK_CAND_ORDER
      }
    }
    if (sel_global || sel_local) {
      const int32_t s0 = sel_off[r], s1 = sel_off[r + 1];
      const int32_t c0 = cand_off ? cand_off[r] : 0, c1 = cand_off ? cand_off[r + 1] : 0;
      for (int32_t j = s0 + (int32_t)threadIdx.x; j < s1; j += kTopkThreads) {
        const int32_t gsel = sel_global ? sel_global[j] : 0;
        if (sel_global) {
          if (gsel < t0 || gsel >= t1) f |= 4;                // CB_CHECK_SEL_RANGE
          if (j > 0 && sel_global[j - 1] >= gsel) f |= 8;     // CB_CHECK_SEL_ORDER (whole batch)
        }
        if (sel_local) {
          const int32_t l = sel_local[j];
          if (l < c0 || l >= c1) f |= 16;                     // CB_CHECK_LOCAL_RANGE
          else if (cand_idx && sel_global && cand_idx[l] != gsel) f |= 32;  // CB_CHECK_LOCAL_MISMATCH
        }
      }
    }
  }
  if (f) atomicOr(&s_flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *flags = s_flags;
}

hipError_t launch_check_indices(const int32_t *tok_off, const int32_t *cand_off,
                                const int32_t *sel_off, int32_t n_req, const int32_t *cand_idx,
                                const int32_t *sel_local, const int32_t *sel_global,
                                int32_t *flags, hipStream_t stream) {
  hipLaunchKernelGGL(check_indices_kernel, dim3(1), dim3(kTopkThreads), 0, stream, tok_off,
                     cand_off, sel_off, n_req, cand_idx, sel_local, sel_global, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fuse, [Derivations, "形式化"]: row sel_global[s] of K/V takes row
// sel_local[s] of the recomputed tensors.  16-byte copies; a row is covered
// by consecutive threads so every access is a contiguous run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fuse_kernel(
    uint4 *__restrict__ k_fused, uint4 *__restrict__ v_fused,
    const uint4 *__restrict__ k_new_c, const uint4 *__restrict__ v_new_c,
    const int32_t *__restrict__ sel_local, const int32_t *__restrict__ sel_global,
    int64_t k_total, int32_t row_vec, uint32_t *__restrict__ clear, int64_t n_clear) {
  const int64_t total = k_total * row_vec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = first; i < n_clear; i += stride) clear[i] = 0;
  for (int64_t i = first; i < total; i += stride) {
    const int64_t s = i / row_vec;
    const int c = (int)(i - s * row_vec);
    const int64_t src = (int64_t)sel_local[s] * row_vec + c;
    const int64_t dst = (int64_t)sel_global[s] * row_vec + c;
    k_fused[dst] = k_new_c[src];
    v_fused[dst] = v_new_c[src];
  }
}

hipError_t launch_fuse(void *k_fused, void *v_fused, const void *k_new_c, const void *v_new_c,
                       const int32_t *sel_local, const int32_t *sel_global, int64_t k_total,
                       int32_t row_bytes, uint32_t *clear, int64_t n_clear, hipStream_t stream) {
  const int32_t row_vec = row_bytes / 16;
  const int64_t total = k_total * row_vec;
  if (total == 0 && n_clear == 0) return hipSuccess;
  int64_t blocks = (std::max(total, n_clear) + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(fuse_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4 *)k_fused,
                     (uint4 *)v_fused, (const uint4 *)k_new_c, (const uint4 *)v_new_c, sel_local,
                     sel_global, k_total, row_vec, clear, n_clear);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotate-or-replace: the re-rotation and the fuse in one pass after the
// selection.  [Derivations, "形式化"] keeps the cached row of every token
// outside S and takes the recomputed row for every token in S, so a row of
// S need not be re-rotated ([Derivations, "CacheBlend 中的应用"]) first:
//   K[t] = t in S ? K_new_c[local(t)] : R_delta(t) K[t],
//   V[t] = t in S ? V_new_c[local(t)] : V[t].
// The re-rotation's token ranges and units are reused.  A workgroup finds the
// entries of S in its range with one 64-ary search of the ascending
// sel_global by its first wave (a ballot per level), maps them in LDS, and
// each unit then copies its two 16-byte pieces of a new K and V row, or
// turns its pairs of a kept K row by the same arithmetic as rerotate_kernel.
// Like the fuse launch it also zeroes clear[0 .. n_clear).
// ---------------------------------------------------------------------------
constexpr int kFuseMapMax = 4096;  // tokens per workgroup (rot_geom keeps <= 16 * 256)

// First index i in [0, n) with a[i] >= key (n if none), for an ascending a.
// Every lane of the calling wave takes part and gets the result.  The first
// probe reads the 64 entries around `guess`; when the answer lies inside
// them (the usual case when the entries spread evenly and guess interpolates)
// that single load settles it, otherwise it narrows [lo, hi] for the 64-ary
// search.
__device__ inline int64_t wave_lower_bound(const int32_t *__restrict__ a, int64_t n, int64_t key,
                                           int64_t guess, int lane) {
  int64_t lo = 0, hi = n;  // the answer lies in [lo, hi]
  if (n > 64) {
    int64_t w0 = guess - 32;
    w0 = w0 < 0 ? 0 : (w0 > n - 64 ? n - 64 : w0);
    const int c = __popcll(__ballot((int64_t)a[w0 + lane] < key));  // a prefix of the window
    if (c < 64 && (c > 0 || w0 == 0)) return w0 + c;
    if (c == 64) lo = w0 + 64;
    else hi = w0;
  }
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t p = lo + lane * step;
    const int c = __popcll(__ballot(p < hi && (int64_t)a[p] < key));  // probes below key
    if (c == 0) return lo;
    const int64_t top = lo + (int64_t)c * step;
    lo += (int64_t)(c - 1) * step + 1;
    hi = top < hi ? top : hi;
  }
  const int64_t p = lo + lane;
  return lo + __popcll(__ballot(p < hi && (int64_t)a[p] < key));
}

template <typename T, int STYLE>
__global__ __launch_bounds__(1024) void rerotate_fuse_kernel(
    T *__restrict__ k, T *__restrict__ v, const T *__restrict__ k_new_c,
    const T *__restrict__ v_new_c, const int32_t *__restrict__ delta,
    const int32_t *__restrict__ sel_local, const int32_t *__restrict__ sel_global,
    int64_t k_total, RotGeom gm, RopeTable tab, uint32_t *__restrict__ clear, int64_t n_clear) {
  constexpr int VP = Vec16<T>::N;
  __shared__ int32_t sel_of[kFuseMapMax];
  __shared__ int64_t s_first;
  const int tid = threadIdx.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < n_clear;
       i += (int64_t)gridDim.x * blockDim.x)
    clear[i] = 0;
  const int64_t t_begin = (int64_t)blockIdx.x * gm.tok_per_block;
  const int64_t t_end = t_begin + gm.tok_per_block < gm.n_tok ? t_begin + gm.tok_per_block : gm.n_tok;
  const int n_rows = (int)(t_end - t_begin);
  for (int i = tid; i < n_rows; i += blockDim.x) sel_of[i] = -1;
  if (tid < 64) {
    const int64_t first =
        wave_lower_bound(sel_global, k_total, t_begin, t_begin * k_total / gm.n_tok, tid);
    if (tid == 0) s_first = first;
  }
  __syncthreads();
  // at most n_rows entries of S fall in [t_begin, t_end), all from s_first on
  for (int i = tid; i < n_rows; i += blockDim.x) {
    const int64_t e = s_first + i;
    if (e < k_total) {
      const int64_t g = sel_global[e];
      if (g >= t_begin && g < t_end) sel_of[g - t_begin] = (int32_t)e;
    }
  }
  __syncthreads();
  if (tid >= gm.units_per_row * gm.tok_per_iter) return;
  const int unit = tid % gm.units_per_row;
  const int slot = tid / gm.units_per_row;
  const int head = unit / gm.units_per_head;
  const int j0 = (unit % gm.units_per_head) * VP;
  const int hd = gm.head_dim;
  const int64_t row_elems = (int64_t)(gm.units_per_row / gm.units_per_head) * hd;
  int p0, p1;
  unit_pieces<T, STYLE>(j0, hd, p0, p1);

  double rev[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) rev[i] = tab.rev_per_pos[j0 + i];
  float cs[VP], sn[VP];
  int cur = INT_MIN;
  for (int64_t t = t_begin + slot; t < t_end; t += gm.tok_per_iter) {
    const int64_t off = t * row_elems + (int64_t)head * hd;
    const int32_t e = sel_of[t - t_begin];
    if (e >= 0) {  // a row of S: the recomputed K and V, bit for bit
      const int64_t src = (int64_t)sel_local[e] * row_elems + (int64_t)head * hd;
      const uint4 k0 = *reinterpret_cast<const uint4 *>(k_new_c + src + p0);
      const uint4 k1 = *reinterpret_cast<const uint4 *>(k_new_c + src + p1);
      const uint4 v0 = *reinterpret_cast<const uint4 *>(v_new_c + src + p0);
      const uint4 v1 = *reinterpret_cast<const uint4 *>(v_new_c + src + p1);
      *reinterpret_cast<uint4 *>(k + off + p0) = k0;
      *reinterpret_cast<uint4 *>(k + off + p1) = k1;
      *reinterpret_cast<uint4 *>(v + off + p0) = v0;
      *reinterpret_cast<uint4 *>(v + off + p1) = v1;
      continue;
    }
    const int d = delta[t];
    if (d == 0) continue;  // R_0 = I
    if (d != cur) {
      cur = d;
      unit_trig<VP>(d, rev, cs, sn);
    }
    rotate_unit<T, STYLE>(k + off, k + off, j0, hd, cs, sn, true);
  }
}

template <typename T, int STYLE>
static hipError_t rerotate_fuse_typed(void *k, void *v, const void *k_new_c, const void *v_new_c,
                                      const int32_t *delta, const int32_t *sel_local,
                                      const int32_t *sel_global, int64_t k_total, int64_t n_tok,
                                      int32_t n_kv_heads, int32_t head_dim, const RopeTable &tab,
                                      uint32_t *clear, int64_t n_clear, hipStream_t stream) {
  int64_t blocks;
  const RotGeom gm = rot_geom<T>(n_tok, 1, n_kv_heads, head_dim, blocks);
  if (blocks == 0) return hipSuccess;
  const int threads = gm.units_per_row * gm.tok_per_iter;
  // the LDS map covers a workgroup's tokens; its first wave searches S
  if (gm.tok_per_block > kFuseMapMax || threads < 64 || threads > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rerotate_fuse_kernel<T, STYLE>), dim3((unsigned)blocks), dim3(threads), 0,
                     stream, (T *)k, (T *)v, (const T *)k_new_c, (const T *)v_new_c, delta,
                     sel_local, sel_global, k_total, gm, tab, clear, n_clear);
  return hipGetLastError();
}

hipError_t launch_rerotate_fuse(int dtype, int style, void *k, void *v, const void *k_new_c,
                                const void *v_new_c, const int32_t *delta,
                                const int32_t *sel_local, const int32_t *sel_global,
                                int64_t k_total, int64_t n_tok, int32_t n_kv_heads,
                                int32_t head_dim, const RopeTable &tab, uint32_t *clear,
                                int64_t n_clear, hipStream_t stream) {
#define CB_RF(T, S)                                                                          \
  rerotate_fuse_typed<T, S>(k, v, k_new_c, v_new_c, delta, sel_local, sel_global, k_total, \
                            n_tok, n_kv_heads, head_dim, tab, clear, n_clear, stream)
  if (dtype == kBF16) return style == 0 ? CB_RF(bf16, 0) : CB_RF(bf16, 1);
  return style == 0 ? CB_RF(float, 0) : CB_RF(float, 1);
#undef CB_RF
}

}  // namespace cb

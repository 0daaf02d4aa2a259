// Partial causal GQA attention of the selected rows over the fused cache.
//
// [Derivations] = "数学推导" (CacheBlend math derivations page), section
// "形式化": the selected rows attend with Attention(Q, K_fused, V_fused).
// [KV-blog] = "rag的kvcache问题": section "阶段二：注意力分数计算阶段" (each
// query row only needs its own q and all of K) and section
// "transformer训练与推理并行计算的差异" (causal mask: no key after the query).
#include <cmath>

#include "cb_device.hpp"
#include "cb_launch.hpp"

namespace cb {

// ---------------------------------------------------------------------------
// MFMA kernel (bf16, head_dim HD in {32, 64, 128}).
//
// A workgroup of 4 waves owns one query tile of 64 query vectors (R selected
// rows x G query heads of one KV group g, R = 64 / G) and streams the keys
// [request start, last row of the tile] through LDS in tiles of 64 keys.
// Each wave owns 16 query vectors.  Scores are computed transposed,
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on the M side, queries on
// the N side), so a lane's accumulators all belong to one query column: the
// online-softmax statistics of that query live in the lane (and its three
// partner lanes l^16, l^32, l^48), and the probabilities feed the second
// product O^T = V^T P^T directly as the B operand with no shuffle.  V is
// transposed on its way into LDS (pairs of keys packed per 32-bit store).
// Blocks are ordered so that blockIdx % Hkv is the KV head: the round-robin
// dispatch over the 8 XCDs then keeps each head's K/V in one XCD's L2 when
// Hkv = 8, and the latest (longest) tiles start first.
// ---------------------------------------------------------------------------
constexpr int kKeyTile = 64;

template <int HD>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    bf16 *__restrict__ out, const bf16 *__restrict__ q_c,
    const int32_t *__restrict__ sel_local, const int32_t *__restrict__ sel_global,
    const bf16 *__restrict__ k_fused, const bf16 *__restrict__ v_fused,
    const int32_t *__restrict__ tok_off, const int32_t *__restrict__ sel_off,
    int32_t n_req, int32_t hq, int32_t hkv, int32_t group, int32_t rows_per_tile,
    int32_t n_tiles, float scale_log2) {
  constexpr int KS = HD + 8;         // LDS row stride of the K tile (elements)
  constexpr int VS = kKeyTile + 8;   // LDS row stride of the V^T tile
  constexpr int NST = HD / 32;       // 32-wide contraction steps over head_dim
  constexpr int NDT = HD / 16;       // 16-row output tiles over head_dim
  __shared__ __attribute__((aligned(16))) bf16 ks[kKeyTile * KS];
  __shared__ __attribute__((aligned(16))) bf16 vt[HD * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x % hkv;
  const int tile_rank = n_tiles - 1 - (int)(blockIdx.x / hkv);

  // Locate this tile's request and first selected row.
  int r = 0, base = 0, s0 = 0, ns = 0;
  for (r = 0; r < n_req; ++r) {
    const int kr = sel_off[r + 1] - sel_off[r];
    const int nt = (kr + rows_per_tile - 1) / rows_per_tile;
    if (tile_rank < base + nt) {
      s0 = sel_off[r] + (tile_rank - base) * rows_per_tile;
      ns = min(rows_per_tile, sel_off[r + 1] - s0);
      break;
    }
    base += nt;
  }
  const int lo = tok_off[r];
  const int p_last = sel_global[s0 + ns - 1];

  // This lane's query column.
  const int col = lane & 15, grp = lane >> 4;
  const int qv = wave * 16 + col;
  const int row = qv / group, hh = qv - row * group;
  const bool qvalid = row < ns;
  const int s = s0 + (qvalid ? row : 0);
  const int p_q = qvalid ? sel_global[s] : lo;  // padding columns see one key
  const int h = g * group + hh;

  bf16x8 qreg[NST];
  {
    const bf16 *qp = q_c + ((int64_t)sel_local[s] * hq + h) * HD + 8 * grp;
#pragma unroll
    for (int st = 0; st < NST; ++st) qreg[st] = *reinterpret_cast<const bf16x8 *>(qp + 32 * st);
  }

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t rs = (int64_t)hkv * HD;  // packed row stride of K/V
  const bf16 *kbase = k_fused + (int64_t)g * HD;
  const bf16 *vbase = v_fused + (int64_t)g * HD;
  const int n_kt = (p_last - lo + kKeyTile) / kKeyTile;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = lo + kt * kKeyTile;
    // Stage K[k0 .. k0+63][g][:] row-major (zeros past the last key).
    for (int c = tid; c < kKeyTile * HD / 8; c += 256) {
      const int key = c / (HD / 8), c8 = c - key * (HD / 8);
      bf16x8 val = {};
      if (k0 + key <= p_last)
        val = *reinterpret_cast<const bf16x8 *>(kbase + (int64_t)(k0 + key) * rs + c8 * 8);
      *reinterpret_cast<bf16x8 *>(ks + key * KS + c8 * 8) = val;
    }
    // Stage V^T: two keys per thread, packed as 32-bit (key, key+1) pairs.
    for (int c = tid; c < (kKeyTile / 2) * (HD / 8); c += 256) {
      const int kp = c / (HD / 8), c8 = c - kp * (HD / 8);
      const int key0 = 2 * kp;
      bf16x8 a = {}, b = {};
      if (k0 + key0 <= p_last)
        a = *reinterpret_cast<const bf16x8 *>(vbase + (int64_t)(k0 + key0) * rs + c8 * 8);
      if (k0 + key0 + 1 <= p_last)
        b = *reinterpret_cast<const bf16x8 *>(vbase + (int64_t)(k0 + key0 + 1) * rs + c8 * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 pr = {a[e], b[e]};
        *reinterpret_cast<bf16x2 *>(vt + (c8 * 8 + e) * VS + key0) = pr;
      }
    }
    __syncthreads();

    // S^T tile: sacc[t][i] = score(key k0 + 16t + 4grp + i, query col).
    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + (16 * t + col) * KS + 32 * st + 8 * grp);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[st], sacc[t], 0, 0, 0);
      }
    }

    // Scale (base-2 logits), causal mask, online softmax.
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * t + 4 * grp + i;
        float v = sacc[t][i] * scale_log2;
        if (key > p_q) v = -INFINITY;
        sacc[t][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);  // finite: key `lo` is visible to every column
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    bf16 pb[16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sacc[t][i] - m_new);
        psum += p;
        pb[4 * t + i] = (bf16)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T over two 32-key halves.
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 bp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bp[i] = pb[4 * (2 * kh) + i];
        bp[4 + i] = pb[4 * (2 * kh + 1) + i];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16 *vrow = vt + (16 * dt + col) * VS + 32 * kh + 4 * grp;
        const bf16x4 lo4 = *reinterpret_cast<const bf16x4 *>(vrow);
        const bf16x4 hi4 = *reinterpret_cast<const bf16x4 *>(vrow + 16);
        bf16x8 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = lo4[i]; a[4 + i] = hi4[i]; }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (qvalid) {
    const float inv = 1.f / l_run;
    bf16 *op = out + ((int64_t)s * hq + h) * HD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (bf16)(o[dt][i] * inv);
      *reinterpret_cast<bf16x4 *>(op + 16 * dt + 4 * grp) = w;
    }
  }
}

int attn_mfma_rows_per_tile(int dtype, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (dtype != kBF16) return 0;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return 0;
  const int group = n_q_heads / n_kv_heads;
  if (group < 1 || group > 64 || 64 % group != 0) return 0;
  return 64 / group;
}

hipError_t launch_attn_mfma(const AttnArgs &a, int32_t rows_per_tile, int32_t n_tiles,
                            hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  const int group = a.n_q_heads / a.n_kv_heads;
  const float scale_log2 = a.softmax_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)((int64_t)n_tiles * a.n_kv_heads)), block(256);
#define CB_ATTN_ARGS                                                                         \
  (bf16 *)a.out, (const bf16 *)a.q_c, a.sel_local, a.sel_global, (const bf16 *)a.k_fused, \
      (const bf16 *)a.v_fused, a.tok_off, a.sel_off, a.n_req, a.n_q_heads, a.n_kv_heads,  \
      group, rows_per_tile, n_tiles, scale_log2
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL(attn_mfma_kernel<32>, grid, block, 0, stream, CB_ATTN_ARGS); break;
    case 64: hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, block, 0, stream, CB_ATTN_ARGS); break;
    default: hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, block, 0, stream, CB_ATTN_ARGS); break;
  }
#undef CB_ATTN_ARGS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plain kernel for every other geometry (fp32 storage, head_dim 16, group
// sizes that do not divide 64): one wave per (selected row, query head),
// 64 keys per step (one per lane), online softmax, fp32 throughout.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline float ld(const T *p) { return (float)*p; }

template <typename T>
__global__ __launch_bounds__(64) void attn_simple_kernel(
    T *__restrict__ out, const T *__restrict__ q_c, const int32_t *__restrict__ sel_local,
    const int32_t *__restrict__ sel_global, const T *__restrict__ k_fused,
    const T *__restrict__ v_fused, const int32_t *__restrict__ tok_off,
    const int32_t *__restrict__ sel_off, int32_t n_req, int32_t hq, int32_t hkv, int32_t hd,
    float scale) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int s = blockIdx.x / hq, h = blockIdx.x - (blockIdx.x / hq) * hq;
  const int g = h / (hq / hkv);
  int r = 0;
  while (r < n_req - 1 && s >= sel_off[r + 1]) ++r;
  const int lo = tok_off[r], hi = sel_global[s];
  const T *q = q_c + ((int64_t)sel_local[s] * hq + h) * hd;
  for (int d = lane; d < hd; d += 64) qs[d] = ld(q + d);
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int u0 = lo; u0 <= hi; u0 += 64) {
    const int u = u0 + lane;
    float sc = -INFINITY;
    if (u <= hi) {
      const T *kr = k_fused + ((int64_t)u * hkv + g) * hd;
      float dot = 0.f;
      for (int d = 0; d < hd; ++d) dot = fmaf(qs[d], ld(kr + d), dot);
      sc = dot * scale;
    }
    const float m_new = fmaxf(m_run, wave_max(sc));
    const float p = (u <= hi) ? expf(sc - m_new) : 0.f;
    const float alpha = expf(m_run - m_new);
    l_run = l_run * alpha + wave_sum(p);
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
    acc0 *= alpha;
    acc1 *= alpha;
    const int nk = min(64, hi - u0 + 1);
    for (int kk = 0; kk < nk; ++kk) {
      const T *vr = v_fused + ((int64_t)(u0 + kk) * hkv + g) * hd;
      const float pk = ps[kk];
      if (lane < hd) acc0 = fmaf(pk, ld(vr + lane), acc0);
      if (lane + 64 < hd) acc1 = fmaf(pk, ld(vr + lane + 64), acc1);
    }
    m_run = m_new;
  }
  T *op = out + ((int64_t)s * hq + h) * hd;
  if (lane < hd) op[lane] = (T)(acc0 / l_run);
  if (lane + 64 < hd) op[lane + 64] = (T)(acc1 / l_run);
}

hipError_t launch_attn_simple(int dtype, const AttnArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.k_total * a.n_q_heads;
  if (blocks == 0) return hipSuccess;
  if (dtype == kBF16)
    hipLaunchKernelGGL(attn_simple_kernel<bf16>, dim3((unsigned)blocks), dim3(64), 0, stream,
                       (bf16 *)a.out, (const bf16 *)a.q_c, a.sel_local, a.sel_global,
                       (const bf16 *)a.k_fused, (const bf16 *)a.v_fused, a.tok_off, a.sel_off,
                       a.n_req, a.n_q_heads, a.n_kv_heads, a.head_dim, a.softmax_scale);
  else
    hipLaunchKernelGGL(attn_simple_kernel<float>, dim3((unsigned)blocks), dim3(64), 0, stream,
                       (float *)a.out, (const float *)a.q_c, a.sel_local, a.sel_global,
                       (const float *)a.k_fused, (const float *)a.v_fused, a.tok_off, a.sel_off,
                       a.n_req, a.n_q_heads, a.n_kv_heads, a.head_dim, a.softmax_scale);
  return hipGetLastError();
}

}  // namespace cb

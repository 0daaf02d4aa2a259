// Partial causal GQA attention of the selected rows over the fused cache.
//
// [Derivations] = "数学推导" (CacheBlend math derivations page), section
// "形式化": the selected rows attend with Attention(Q, K_fused, V_fused).
// [KV-blog] = "rag的kvcache问题": section "阶段二：注意力分数计算阶段" (each
// query row only needs its own q and all of K) and section
// "transformer训练与推理并行计算的差异" (causal mask: no key after the query).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "cb_device.hpp"
#include "cb_launch.hpp"

namespace cb {

// ---------------------------------------------------------------------------
// MFMA kernel (bf16, head_dim HD in {32, 64, 128}).
//
// Work unit = (query tile, KV head g, key chunk).  A query tile holds the
// query vectors of rows_per_tile selected rows of one request times the
// G = Hq/Hkv query heads that read KV head g, so one K/V stream serves all of
// them.  A workgroup of 8 waves (two per SIMD) owns a unit; each wave owns 32
// query vectors.  Keys stream through LDS in tiles of 64.  All products use
// v_mfma_f32_32x32x16_bf16, which on gfx950 sustains about twice the rate of
// the 16x16x32 form.  Lane l of a 32x32 result holds rows
// 8(r/4) + 4(l/32) + r%4 (r = 0..15) of column l%32.
//
//  * Key split KS: with KS = 1 the 8 waves cover 256 query vectors over
//    64-key tiles in 4 LDS stages; with KS = 2 they form two key groups over
//    the same 128 query vectors and 128-key tiles in 2 stages (the same LDS
//    bytes), group h taking keys 64h .. 64h+63 of every tile, so each wave
//    does the same work between two barriers; group 1 hands its (max, sum,
//    O) to group 0 through LDS at the end.  KS = 2 halves the time of a unit
//    over the same keys (the longest unit bounds small launches) without any
//    partial in global memory, at the price of twice the K/V staging per
//    query and a shallower prefetch.
//  * Staging: K and V tiles go global -> LDS with global_load_lds_dwordx4
//    (no registers) through the LDS stages: tile t + stages - 1 is issued
//    while tile t is multiplied.  The LDS tiles are row-major with an XOR
//    swizzle of the 16-byte chunks of each key row (different for K and V)
//    so that the two read patterns below are free of bank conflicts.
//  * S^T = K Q^T (keys on the M side, queries on the N side) in 32-key
//    blocks: a lane's scores all belong to one query column, so the
//    online-softmax statistics stay in the lane and its partner l^32 (pair
//    exchange through v_permlane32_swap), and the
//    probabilities of 16 consecutive keys are 8 consecutive accumulator
//    registers -- already the B operand of the second product.
//  * O^T += V^T P^T in 32-dim blocks.  The A operand (8 keys of one head
//    dimension per lane) comes from gfx950's ds_read_b64_tr_b16: in each
//    16-lane group, lane j points at V[key0 + j/4][d0 + 4(j%4)] and lane i
//    receives V[key0 .. key0+3][d0 + i].
//  * Softmax in base 2 with the scale folded into one FMA; the running max is
//    only raised (and O rescaled) when a column's tile max exceeds it by more
//    than 2^8, so most tiles skip the rescale; tiles that every query of the
//    unit sees in full skip the causal mask.
//
// Long rows with too few tiles to fill the chip are split over key chunks of
// `key_chunk` keys (a multiple of the tile); every working chunk writes its
// partial to the workspace -- O of each query vector divided by its largest
// |O| as fp16, then the running max, running sum and that largest |O| in
// fp32 -- and the last chunk of the tile to arrive merges them (see the end
// of the kernel).  Unsplit units write the output directly.
// Block order: blockIdx % Hkv is the KV head, so with Hkv = 8 the round-robin
// dispatch over the 8 XCDs keeps each head's K/V stream in one XCD's L2.  In
// a request, units go chunk by chunk and, within a chunk, from the last
// (longest) tile to the first: the later chunks of early tiles, which lie
// past their tile's last row and exit at once, come last and do not hold a
// CU while a working unit waits for one.
// ---------------------------------------------------------------------------
struct AttnParams {
  bf16 *out;
  const bf16 *q_c;
  const int32_t *sel_local;
  const int32_t *sel_global;
  const bf16 *k_fused;
  const bf16 *v_fused;
  const int32_t *tok_off;
  const int32_t *sel_off;
  unsigned char *ws;     // split partials, one per workgroup of the launch
  unsigned *cnt;         // arrival counter per (query tile, KV head); zero at launch and at exit
  int32_t n_req, hq, hkv, group, rows_per_tile, key_chunk;
  int32_t spans;         // > 0: balanced decomposition over this many workgroups per KV head
  float scale_log2;
};

// Launch order of the units, passed by value (kernel arguments: the table
// needs no device memory and is captured with the launch).  Sized to the
// launch: kernel arguments travel to the device with every launch, and a
// short launch feels 4 KB of them.
constexpr int kMaxOrder = kAttnMaxOrder;
template <int N>
struct AttnOrder {
  uint32_t e[N];  // units, by their index in the kernel's own order
};

constexpr int kKeyTile = 64;
constexpr int kWaves = 8;              // waves per workgroup, two per SIMD
constexpr int kQT = 32 * kWaves;       // query vectors per unit
constexpr int kStages = 4;             // K/V tiles resident in LDS
constexpr float kNegFloor = -1.0e30f;  // finite start of the running max
constexpr float kRescaleSlack = 8.0f;  // log2 headroom before the max is raised
constexpr int kMaxChunks = 8;          // key chunks per row (split plan bound)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Bytes of one split partial of QT query vectors: fp16 O in fragment order,
// then three fp32 values per query vector (running max, running sum, largest
// |O|).
template <int HD, int QT> constexpr int partial_bytes() { return QT * HD * 2 + 3 * QT * 4; }
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

__device__ inline bf16x4 lds_read_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// Swizzled 16-byte chunk of key row r: physical chunk = logical ^ f(r).
// Chosen so that both read patterns below hit every bank once whether LDS
// serves 128 B per cycle (b128 reads in groups of 8 lanes, b64 in groups of
// 16) or 256 B (groups of 16 and 32).
//  K: b128 reads of 32 consecutive rows (lane l: row l%32) at one logical chunk.
//  V: transpose reads; lane l reads 8 bytes of row 4(l/32) + (l%16)/4 at
//     logical chunk 4*dt + 2*((l/16)%2) + (l%4)/2.
template <int HD> __device__ constexpr int swz_k(int r) {
  if constexpr (HD == 128) return r & 15;
  else if constexpr (HD == 64) return ((r >> 1) & 7) ^ (4 * (r & 1));
  else return ((r >> 2) & 3) ^ (2 * ((r >> 1) & 1));
}
template <int HD> __device__ constexpr int swz_v(int r) {
  if constexpr (HD == 128) return 10 * (r & 1) + 4 * ((r >> 1) & 1);
  else if constexpr (HD == 64) return 2 * (r & 3);
  else return 2 * ((r >> 1) & 1);
}

// Where a unit sits: request r, its query tile and key chunk, the request's
// tile and chunk counts, and the units and tiles of the requests before it.
struct UnitPos {
  int r, tile, chunk, tr, nchunks;
  int64_t ubase, tbase;
};

// Unit u -> its position: within a request, chunk-major, tiles from last to
// first.  Returns false past the last unit.
__device__ inline bool locate_unit(const AttnParams &p, int u, UnitPos &up) {
  int64_t ubase = 0, tbase = 0;
  for (int r = 0; r < p.n_req; ++r) {
    const int kr = p.sel_off[r + 1] - p.sel_off[r];
    const int n = p.tok_off[r + 1] - p.tok_off[r];
    const int tr = (kr + p.rows_per_tile - 1) / p.rows_per_tile;
    const int cr = (int)(((int64_t)n + p.key_chunk - 1) / p.key_chunk);
    const int64_t nu = (int64_t)tr * cr;
    if (u < ubase + nu) {
      const int ul = (int)(u - ubase);
      up.r = r;
      up.chunk = ul / tr;
      up.tile = tr - 1 - (ul - up.chunk * tr);
      up.tr = tr;
      up.nchunks = cr;
      up.ubase = ubase;
      up.tbase = tbase;
      return true;
    }
    ubase += nu;
    tbase += tr;
  }
  return false;
}


// 16 bytes per lane from global memory straight into LDS: lane l writes
// lds_byte + 16 l (gfx950 global_load_lds_dwordx4, LDS base in M0).  Written
// as inline assembly so the compiler, which cannot tell the LDS stages apart,
// does not wait for every copy in flight before each LDS read; the kernel
// waits for its copies itself (waitcnt on the VM counter, then a barrier).
// Nothing else in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const char *base, uint32_t off, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               :: "v"(off), "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Split partials pass between workgroups on different XCDs, whose L2 caches
// are not coherent with each other.  They are stored and loaded only with
// store_agent / load_agent (relaxed agent-scope atomics, performed at the
// coherence point all XCDs share); the arrival counter is such an atomic too.
// So no fence has to write back or invalidate a whole L2 (an agent-scope
// fence does both, and in every workgroup it tripled the launch time).

// Lanes l and l ^ 32 hold the two halves of one query column.  gfx950's
// v_permlane32_swap trades the upper 32 lanes of one register with the lower
// 32 lanes of another; swapping x with itself leaves each lane holding, in
// the two results, x of itself and x of lane l ^ 32 -- no LDS round trip
// (a shuffle through ds_bpermute costs one on the path from the scores to
// the exponentials of every tile).
__device__ inline float lane_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float lane_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint32_t lds_addr(const bf16 *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16 *)p;
}


// Compile-time shape of one MFMA attention workgroup.
template <int HD, int KS> struct AttnCfg {
  static_assert(KS == 1 || KS == 2, "key split of 1 or 2 groups");
  static constexpr int QT = kQT / KS;            // query vectors per unit
  static constexpr int WPG = kWaves / KS;        // waves per key group
  static constexpr int KT = kKeyTile * KS;       // keys per tile: 64 per key group
  static constexpr int STAGES = kStages / KS;    // tiles resident in LDS (the same bytes)
  static constexpr int NSB = 2;                  // 32-key blocks per wave and tile
  static constexpr int NKS = HD / 16;            // 16-wide contraction steps of S over head_dim
  static constexpr int NDT = HD / 32;            // 32-dim output blocks
  static constexpr int CPR = HD / 8;             // 16-byte chunks per key row
  static constexpr int TILE = KT * HD;           // elements per tensor per stage
  static constexpr int NI = TILE / 512;          // 1 KiB DMA instructions per tensor per tile
  static constexpr int DMA_WAVES = NI < kWaves ? NI : kWaves;
  static constexpr int IPW = NI / DMA_WAVES;     // per issuing wave and tensor
  static constexpr int PER_TILE = 2 * IPW;       // vector-memory ops per tile and issuing wave
};

// One piece of attention work: query tile `tile` of request `r` (KV head g)
// over the keys [k_begin, k_end), k_end <= p_last + 1.  With n_active == 1 the
// piece covers the tile's whole row and writes the output; otherwise it
// stores its partial at `own`, and the last of the tile's n_active pieces to
// arrive (counter `item` of head g) merges all of them, in piece order, and
// writes the output.  Piece c's partial: part0 for c == 0, else
// part1 + (c - 1) * part_stride.
struct Piece {
  int r, tile, s0, ns, lo, p_first, p_last, k_begin, k_end, n_active;
  int64_t item;
  unsigned char *own;
  const unsigned char *part0, *part1;
  int64_t part_stride;
};

template <int HD, int KS>
__device__ __attribute__((always_inline)) void attn_piece(
    const AttnParams &p, const int g, const Piece &pc,
    bf16 (*kst)[AttnCfg<HD, KS>::TILE], bf16 (*vst)[AttnCfg<HD, KS>::TILE], int &s_last) {
  using C = AttnCfg<HD, KS>;
  constexpr int QT = C::QT, WPG = C::WPG, KT = C::KT, STAGES = C::STAGES, NSB = C::NSB;
  constexpr int NKS = C::NKS, NDT = C::NDT, CPR = C::CPR, TILE = C::TILE;
  constexpr int DMA_WAVES = C::DMA_WAVES, IPW = C::IPW, PER_TILE = C::PER_TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int kg = wave / WPG;              // key group: keys 64kg .. 64kg+63 of each tile
  const int s0 = pc.s0, ns = pc.ns, lo = pc.lo, p_first = pc.p_first, p_last = pc.p_last;
  const int k_begin = pc.k_begin, k_end = pc.k_end;
  const int n_kt = (k_end - k_begin + KT - 1) / KT;
  (void)lo;
  phase_barrier();  // a previous piece of this workgroup is done with the LDS stages

  // DMA slots of this wave: instruction i writes 64 consecutive 16-byte chunks
  // of the tile; lane -> (row, physical chunk) -> logical chunk.  Rows past
  // the tile's last key are clamped onto it (their scores are masked).
  const int64_t rs = (int64_t)p.hkv * HD;
  const bool dma_wave = wave < DMA_WAVES;
  int dma_row[IPW];
  uint32_t dma_ko[IPW], dma_vo[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int pos = ((dma_wave ? wave : 0) * IPW + i) * 64 + lane;
    const int row = pos / CPR, q = pos - row * CPR;
    dma_row[i] = row;
    dma_ko[i] = (uint32_t)((row * rs + (q ^ swz_k<HD>(row)) * 8) * 2);
    dma_vo[i] = (uint32_t)((row * rs + (q ^ swz_v<HD>(row)) * 8) * 2);
  }
  const char *kbase = (const char *)(p.k_fused + (int64_t)g * HD);
  const char *vbase = (const char *)(p.v_fused + (int64_t)g * HD);
  auto issue_tile = [&](int t) {
    if (!dma_wave) return;
    const int k0 = k_begin + t * KT;
    const int64_t tb = (int64_t)k0 * rs * 2;
    const bool clamp = k0 + KT - 1 > p_last;
    const uint32_t kd = lds_addr(kst[t % STAGES]) + wave * IPW * 1024;
    const uint32_t vd = lds_addr(vst[t % STAGES]) + wave * IPW * 1024;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      uint32_t back = 0;
      if (clamp && k0 + dma_row[i] > p_last) back = (uint32_t)((k0 + dma_row[i] - p_last) * rs * 2);
      dma16(kbase + tb, dma_ko[i] - back, kd + i * 1024);
      dma16(vbase + tb, dma_vo[i] - back, vd + i * 1024);
    }
  };

  // This lane's query column.  Padding columns (past the tile's last row)
  // see every key; their results are dropped.
  const int qv = (wave - kg * WPG) * 32 + col;
  const int qrow = qv / p.group, qhh = qv - qrow * p.group;
  const bool qvalid = qrow < ns;
  int p_q;
  bf16x8 qreg[NKS];  // Q^T fragment of step s: dims 16s + 8*half .. +7
  {
    const int s = s0 + (qvalid ? qrow : 0);
    p_q = qvalid ? p.sel_global[s] : p_last;
    const bf16 *qp = p.q_c + ((int64_t)p.sel_local[s] * p.hq + g * p.group + qhh) * HD + 8 * half;
#pragma unroll
    for (int st = 0; st < NKS; ++st) qreg[st] = *reinterpret_cast<const bf16x8 *>(qp + 16 * st);
  }
  for (int t = 0; t < STAGES - 1 && t < n_kt; ++t) issue_tile(t);

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m_run = kNegFloor, l_run = 0.f;

  // LDS read offsets of this lane (elements within a stage buffer).
  // K fragment of step st for key block sb: koff[st] + sb*32*HD.
  // V^T fragment of dim block dt, 16-key step c, second 4 keys: voff[dt] +
  // c*16*HD (+ 8*HD).
  int koff[NKS], voff[NDT];
#pragma unroll
  for (int st = 0; st < NKS; ++st) koff[st] = col * HD + (((2 * st + half) ^ swz_k<HD>(col)) << 3);
  {
    const int q4 = (lane & 15) >> 2;
    const int row = 4 * half + q4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int e = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[dt] = row * HD + (((e >> 3) ^ swz_v<HD>(row)) << 3) + (e & 7);
    }
  }

  // Q (issued first) and tile 0 resident; the later prefetched tiles may stay
  // in flight.  The compiler, which does not count the copies into LDS, adds
  // its own waits before the first uses of Q; it peels them into the first
  // iteration, so the tile loop keeps only the waits below.
  const int ahead0 = min(STAGES - 2, n_kt - 1);  // tiles issued after tile 0
  if (ahead0 >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER_TILE));
  else if (ahead0 == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER_TILE));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = k_begin + kt * KT;
    // Tile kt has landed for this wave's share; the tiles issued after it
    // (up to STAGES - 2 of them) may stay in flight.  The barrier then makes
    // every wave's share visible and tells that all waves are done with tile
    // kt - 1, whose stage is refilled with tile kt + STAGES - 1.
    if (kt > 0) {
      const int ahead = min(kt + STAGES - 2, n_kt - 1) - kt;
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER_TILE));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER_TILE));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    phase_barrier();
    if (kt + STAGES - 1 < n_kt) issue_tile(kt + STAGES - 1);
    const bf16 *ks = kst[kt % STAGES];
    const bf16 *vs = vst[kt % STAGES];

    // S^T: sacc[sb][r] = score(key kg0 + 32sb + 8(r/4) + 4*half + r%4, column)
    // for this wave's key group (kg0 = first key of the group in the tile).
    const int kg0 = k0 + 32 * NSB * kg;
    const bf16 *ksg = ks + NSB * kg * 32 * HD;
    f32x16 sacc[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[sb][e] = 0.f;
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ksg + koff[st] + sb * 32 * HD);
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[st], sacc[sb], 0, 0, 0);
      }
    }
    // Keep four K fragments in flight ahead of the products: left alone, the
    // compiler reads each fragment right before its product and every
    // product waits out an LDS latency (measured: 2-4% of the launch at the
    // 6k to 70B-batch shapes).
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < NKS * NSB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }

    if (kg0 + 32 * NSB - 1 > p_first) {  // causal mask (key blocks past the first row)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kg0 + 32 * sb + 8 * (e >> 2) + 4 * half + (e & 3) > p_q) sacc[sb][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[sb][e]);
    mx = lane_pair_max(mx);
    const float mxs = mx * p.scale_log2;
    const bool raise = mxs > m_run + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = raise ? mxs : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    const float neg_m = -m_run;
    bf16x8 bp[2 * NSB];  // probabilities of keys kg0 + 16c .. kg0 + 16c + 15
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        bp[2 * sb + (e >> 3)][e & 7] =
            (bf16)__builtin_amdgcn_exp2f(fmaf(sacc[sb][e], p.scale_log2, neg_m));
    // The running sum adds the probabilities as they enter the PV product
    // (bf16), two per v_dot2c_f32_bf16, in two independent chains.
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2 * NSB; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ps[i & 1] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{bp[c][2 * i], bp[c][2 * i + 1]},
                                                    one2, ps[i & 1], false);
    l_run += ps[0] + ps[1];

    // O^T += V^T P^T: per 16-key step c, one transposed V fragment per dim block.
    const bf16 *vsg = vs + 2 * NSB * kg * 16 * HD;
#pragma unroll
    for (int c = 0; c < 2 * NSB; ++c) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16 *vp = vsg + voff[dt] + c * 16 * HD;
        const bf16x4 lo4 = lds_read_tr(vp);
        const bf16x4 hi4 = lds_read_tr(vp + 8 * HD);
        const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp[c], o[dt], 0, 0, 0);
      }
    }
  }

  float l = lane_pair_sum(l_run);
  if constexpr (KS == 2) {
    // Key group 1 hands (running max, running sum, O) of its query vectors to
    // group 0 through LDS (the stage buffers are free once every wave is past
    // its last tile): O in fragment order, 16 bytes per lane and store.
    static_assert(STAGES * TILE * 2 >= WPG * NDT * 16 * 64 * 4, "O exchange does not fit");
    float *xo = reinterpret_cast<float *>(&vst[0][0]);
    float *xm = reinterpret_cast<float *>(&kst[0][0]);
    phase_barrier();
    if (kg == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 w = {o[dt][4 * q], o[dt][4 * q + 1], o[dt][4 * q + 2], o[dt][4 * q + 3]};
          *reinterpret_cast<f32x4 *>(xo + 4 * ((((wave - WPG) * NDT + dt) * 4 + q) * 64 + lane)) = w;
        }
      if (half == 0) {
        xm[qv] = m_run;
        xm[QT + qv] = l;
      }
    }
    phase_barrier();
    if (kg == 0) {
      const float mb = xm[qv], lb = xm[QT + qv];
      const float mm = fmaxf(m_run, mb);
      const float wa = __builtin_amdgcn_exp2f(m_run - mm), wb = __builtin_amdgcn_exp2f(mb - mm);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 w = *reinterpret_cast<const f32x4 *>(
              xo + 4 * (((wave * NDT + dt) * 4 + q) * 64 + lane));
#pragma unroll
          for (int i = 0; i < 4; ++i) o[dt][4 * q + i] = fmaf(o[dt][4 * q + i], wa, w[i] * wb);
        }
      l = fmaf(l, wa, lb * wb);
      m_run = mm;
    }
  }
  // Split over keys: every working chunk of the tile stores its partial;
  // the last to arrive merges all of them and writes the output.  A tile
  // whose rows all lie in its first chunk has one working unit and no merge.
  const int n_active = pc.n_active;
  // The merge of a split tile: with key split 2 both wave groups take part,
  // each on half of the dim blocks of its query vectors (one dim block:
  // group 0 alone); with key split 1 every wave on its own vectors.
  constexpr int MSPLIT = (KS == 2 && NDT >= 2) ? 2 : 1;
  constexpr int MDT = NDT / MSPLIT;          // dim blocks merged per wave
  constexpr int MCH = MDT * 4 <= 8 ? 4 : 2;  // chunks whose loads are in flight at once
  const bool merging = KS == 1 || MSPLIT == 2 || kg == 0;
  const int dt_lo = MSPLIT == 2 ? kg * MDT : 0;
  bool merged = false;
  if (n_active > 1) {
    if (kg == 0) {
      // Partial in fragment order: store (dt, q) of wave w writes 64 lanes x 8
      // contiguous bytes at fp16x4 index ((w*NDT + dt)*4 + q)*64 + lane.  Each
      // query vector's O is divided by its largest |O| (the two lanes l and
      // l ^ 32 hold its dims), so fp16 keeps 11 significant bits of every
      // value whatever the scale of V; the merge multiplies it back.
      unsigned char *w = pc.own;
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o[dt][e]));
      amax = lane_pair_max(amax);
      const float inv_amax = amax > 0.f ? 1.f / amax : 0.f;
      uint64_t *wo = reinterpret_cast<uint64_t *>(w);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f16x4 h;
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = (_Float16)(o[dt][4 * q + i] * inv_amax);
          store_agent(wo + (((wave * NDT + dt) * 4 + q) << 6) + lane, __builtin_bit_cast(uint64_t, h));
        }
      if (half == 0) {
        uint32_t *meta = reinterpret_cast<uint32_t *>(w + QT * HD * 2);
        store_agent(meta + qv, __builtin_bit_cast(uint32_t, m_run));
        store_agent(meta + QT + qv, __builtin_bit_cast(uint32_t, l));
        store_agent(meta + 2 * QT + qv, __builtin_bit_cast(uint32_t, amax));
      }
    }
    // Arrival: every store of the partial has completed at the coherence
    // point shared by all XCDs before the arrival is counted; the workgroup
    // that brings the count to n_active goes on.  It is the last to touch
    // the counter in this launch, so it sets it back to zero: every launch
    // leaves its counters as it needs to find them.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    phase_barrier();
    if (tid == 0) {
      unsigned *const cnt = p.cnt + pc.item * p.hkv + g;
      const unsigned prev =
          __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)(n_active - 1);
      if (s_last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    phase_barrier();
    if (!s_last) return;  // uniform
    merged = true;
    // Merge every piece's stored partial, this one's included, in piece
    // order: the result does not depend on which piece arrived last.
    if (merging) {
      auto part = [&](int c) -> const unsigned char * {
        return c == 0 ? pc.part0 : pc.part1 + (int64_t)(c - 1) * pc.part_stride;
      };
      const int fw = wave - kg * WPG;  // query block of this wave in the fragment order
      // One round of loads for up to MCH chunks: the running max, running
      // sum and largest |O| of every chunk, then the first MCH chunks' O
      // fragments (issued before any of them is used), then a round per
      // further MCH chunks.  O of the dim blocks D0 .. D0 + MDT - 1 adds up in
      // chunk order; all indices are unrolled constants, so nothing leaves
      // the registers.
      auto merge_dims = [&](auto d0) {
        constexpr int D0 = decltype(d0)::value;
        float mc[kMaxChunks], lc[kMaxChunks], ac[kMaxChunks];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          mc[c] = kNegFloor;
          lc[c] = ac[c] = 0.f;
          if (c < n_active) {
            const uint32_t *mt =
                reinterpret_cast<const uint32_t *>(part(c) + QT * HD * 2);
            mc[c] = __builtin_bit_cast(float, load_agent(mt + qv));
            lc[c] = __builtin_bit_cast(float, load_agent(mt + QT + qv));
            ac[c] = __builtin_bit_cast(float, load_agent(mt + 2 * QT + qv));
          }
        }
        f16x4 h[MCH][MDT * 4];
        auto load_group = [&](int c0) {
#pragma unroll
          for (int j = 0; j < MCH; ++j) {
            if (c0 + j < n_active) {
              const uint64_t *src = reinterpret_cast<const uint64_t *>(part(c0 + j));
#pragma unroll
              for (int dl = 0; dl < MDT; ++dl)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  h[j][dl * 4 + q] = __builtin_bit_cast(
                      f16x4, load_agent(src + (((fw * NDT + D0 + dl) * 4 + q) << 6) + lane));
            }
          }
        };
        load_group(0);
        float mx = kNegFloor;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) mx = fmaxf(mx, mc[c]);
        float wgt[kMaxChunks];
        l = 0.f;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
          wgt[c] = c < n_active ? __builtin_amdgcn_exp2f(mc[c] - mx) : 0.f;
          l = fmaf(lc[c], wgt[c], l);
          wgt[c] *= ac[c];
        }
#pragma unroll
        for (int dl = 0; dl < MDT; ++dl) o[D0 + dl] = 0.f;
#pragma unroll
        for (int c0 = 0; c0 < kMaxChunks; c0 += MCH) {
          if (c0 < n_active) {
            if (c0 > 0) load_group(c0);
#pragma unroll
            for (int j = 0; j < MCH; ++j) {
              if (c0 + j < n_active) {
#pragma unroll
                for (int dl = 0; dl < MDT; ++dl)
#pragma unroll
                  for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      o[D0 + dl][4 * q + i] =
                          fmaf((float)h[j][dl * 4 + q][i], wgt[c0 + j], o[D0 + dl][4 * q + i]);
              }
            }
          }
        }
      };
      if (dt_lo == 0) merge_dims(std::integral_constant<int, 0>{});
      else merge_dims(std::integral_constant<int, MDT>{});
    }
  }

  // Output through LDS (the K stage buffers are free once every wave is past
  // its last tile): each wave holding results writes its normalised bf16
  // rows (16-byte chunk index XOR-swizzled by the query vector against bank
  // conflicts), then the workgroup stores 16-byte chunks in output order --
  // the G query heads of one selected row are adjacent in `out`, so a wave
  // writes whole 1 KiB runs instead of 8 bytes per lane 256 bytes apart.
  // Unmerged, key group 0 holds every dim block; merged, each merging wave
  // holds its own.
  constexpr int CPQ = HD / 8;  // 16-byte chunks per query vector
  bf16 *stage = &kst[0][0];
  static_assert(STAGES * TILE >= QT * HD, "output staging does not fit");
  phase_barrier();
  const bool writer = merged ? merging : kg == 0;
  const int w_lo = merged ? dt_lo : 0, w_hi = merged ? dt_lo + MDT : NDT;
  if (writer) {
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt < w_lo || dt >= w_hi) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (bf16)(o[dt][4 * q + i] * inv);
        const int cq = (4 * dt + q) ^ (qv & (CPQ - 1));
        *reinterpret_cast<bf16x4 *>(stage + qv * HD + 8 * cq + 4 * half) = w;
      }
    }
  }
  phase_barrier();
  for (int c = tid; c < QT * CPQ; c += 64 * kWaves) {
    const int v = c / CPQ, part = c - v * CPQ;
    const int vrow = v / p.group, vh = v - vrow * p.group;
    if (vrow < ns)
      *reinterpret_cast<uint4 *>(p.out + ((int64_t)(s0 + vrow) * p.hq + g * p.group + vh) * HD +
                                 8 * part) =
          *reinterpret_cast<const uint4 *>(stage + v * HD + 8 * (part ^ (v & (CPQ - 1))));
  }
}

// Tables of the balanced decomposition: tiles per request, then each query
// tile's 64-key tiles laid end to end (exclusive prefix sums), in LDS.
constexpr int kStreamMaxRequests = 1024;
constexpr int kStreamMaxTiles = 2048;

// Exclusive prefix sum of a[0 .. n) in place (n <= 4 * 512), a[n] = total;
// every thread of the 512-thread workgroup takes part (the entries may have
// been written by any thread just before).  tmp: kWaves words.
__device__ inline void block_scan_exclusive(uint32_t *a, int n, uint32_t *tmp) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __syncthreads();  // every thread's writes of a are visible
  uint32_t v[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * t + q;
    v[q] = i < n ? a[i] : 0u;
    s += v[q];
  }
  uint32_t x = s;  // inclusive scan over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;  // tmp's readers of a previous scan passed its last barrier
  __syncthreads();
  uint32_t run = x - s, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) run += tmp[w];
    total += tmp[w];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * t + q;
    if (i < n) a[i] = run;
    run += v[q];
  }
  if (t == 0) a[n] = total;
  __syncthreads();
}

// Largest i in [0, n) with a[i] <= x, for an ascending a with a[0] <= x.
__device__ inline int upper_index(const uint32_t *a, int n, uint32_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Balanced decomposition (key split 1): the 64-key tiles of all query tiles
// of KV head g, laid end to end in request and tile order, are cut into
// p.spans equal spans of S tiles, one per workgroup (S at least a seventh of
// the longest row, so a row is cut into at most 8 pieces).  A workgroup
// computes the layout itself (one selected-row position per query tile) and
// runs each piece of its span: query tiles inside the span whole, the ones
// cut by its ends as pieces whose partials merge like key chunks.  Partial
// slots: two per workgroup, slot 1 for the piece of a tile that starts inside
// the span, slot 0 for the first piece.
template <int HD>
__device__ __attribute__((always_inline)) void attn_stream(
    const AttnParams &p, const int g, bf16 (*kst)[AttnCfg<HD, 1>::TILE],
    bf16 (*vst)[AttnCfg<HD, 1>::TILE], int &s_last, uint32_t *tb, uint32_t *gt, uint32_t *tmp,
    uint32_t &s_maxn) {
  const int tid = threadIdx.x;
  const int rpt = p.rows_per_tile, n_req = p.n_req;
  const uint32_t w = blockIdx.x / p.hkv, n_spans = (uint32_t)p.spans;
  if (n_req > kStreamMaxRequests) return;  // uniform; the host plans within the tables
  // query tiles per request -> tb (exclusive prefix), tb[n_req] = all tiles
  for (int r = tid; r < n_req; r += 64 * kWaves) {
    const int kr = p.sel_off[r + 1] - p.sel_off[r];
    tb[r] = (uint32_t)((kr + rpt - 1) / rpt);
  }
  if (tid == 0) s_maxn = 0;
  block_scan_exclusive(tb, n_req, tmp);
  const int n_items = (int)tb[n_req];
  if (n_items > kStreamMaxTiles) return;  // uniform; the host plans within the tables
  // 64-key tiles of each query tile: its last selected row's position in the request
  // (the request of tile i: the last r with tb[r] <= i, so requests without
  // selected rows, which repeat the previous tb value, are passed over)
  for (int i = tid; i < n_items; i += 64 * kWaves) {
    const int r = upper_index(tb, n_req, (uint32_t)i);
    const int tile = i - (int)tb[r];
    const int s0 = p.sel_off[r], kr = p.sel_off[r + 1] - s0;
    if (tile < 0 || tile * rpt >= kr) {  // cannot happen with the table above; never read outside
      gt[i] = 1;
      continue;
    }
    const int last = s0 + min((tile + 1) * rpt, kr) - 1;
    const uint32_t n = (uint32_t)((p.sel_global[last] - p.tok_off[r]) / kKeyTile + 1);
    gt[i] = n;
    atomicMax(&s_maxn, n);
  }
  block_scan_exclusive(gt, n_items, tmp);
  const uint32_t total = gt[n_items], maxn = s_maxn;
  const uint32_t span = max((total + n_spans - 1) / n_spans, (maxn + 6) / 7);
  const uint32_t t0 = w * span, t1 = min(total, t0 + span);
  if (t0 >= t1) return;  // uniform: nothing left for this span
  constexpr int64_t UNIT = partial_bytes<HD, kQT>();
  auto slot = [&](uint32_t ww, int sl) {
    return p.ws + (((int64_t)ww * p.hkv + g) * 2 + sl) * UNIT;
  };
  for (int i = upper_index(gt, n_items, t0); i < n_items && gt[i] < t1; ++i) {
    const uint32_t gi = gt[i], ni = gt[i + 1] - gi;
    const uint32_t a = max(t0, gi) - gi, b = min(t1, gi + ni) - gi;
    const int r = upper_index(tb, n_req, (uint32_t)i);
    Piece pc;
    pc.r = r;
    pc.tile = i - (int)tb[r];
    pc.s0 = p.sel_off[r] + pc.tile * rpt;
    pc.ns = min(rpt, p.sel_off[r + 1] - pc.s0);
    pc.lo = p.tok_off[r];
    pc.p_first = p.sel_global[pc.s0];
    pc.p_last = p.sel_global[pc.s0 + pc.ns - 1];
    pc.k_begin = pc.lo + kKeyTile * (int)a;
    pc.k_end = min(pc.p_last + 1, pc.lo + kKeyTile * (int)b);
    const uint32_t wa = gi / span, wb = (gi + ni - 1) / span;
    // (wb < n_spans and at most kMaxChunks pieces follow from the layout above;
    // the check keeps every partial slot and merge inside the workspace)
    if (wb >= n_spans || wb - wa >= (uint32_t)kMaxChunks) return;  // uniform
    pc.n_active = (int)(wb - wa + 1);
    pc.item = i;
    pc.own = pc.n_active > 1 ? slot(w, t0 < gi ? 1 : 0) : nullptr;
    pc.part0 = pc.n_active > 1 ? slot(wa, wa * span < gi ? 1 : 0) : nullptr;
    pc.part1 = pc.n_active > 1 ? slot(wa + 1, 0) : nullptr;
    pc.part_stride = (int64_t)p.hkv * 2 * UNIT;
    attn_piece<HD, 1>(p, g, pc, kst, vst, s_last);
  }
}

// Unit u of the (query tile, key chunk) decomposition, KV head g.  Unit
// ubase + c * tr + (tr - 1 - tile) of a request is chunk c of its query tile
// `tile`; its partial (when the tile is split) sits in slot u * hkv + g.
template <int HD, int KS>
__device__ __attribute__((always_inline)) void attn_unit(
    const AttnParams &p, const int u, const int g, bf16 (*kst)[AttnCfg<HD, KS>::TILE],
    bf16 (*vst)[AttnCfg<HD, KS>::TILE], int &s_last) {
  using C = AttnCfg<HD, KS>;
  UnitPos up;
  if (!locate_unit(p, u, up)) return;
  Piece pc;
  pc.r = up.r;
  pc.tile = up.tile;
  pc.s0 = p.sel_off[pc.r] + pc.tile * p.rows_per_tile;
  pc.ns = min(p.rows_per_tile, p.sel_off[pc.r + 1] - pc.s0);
  pc.lo = p.tok_off[pc.r];
  pc.p_first = p.sel_global[pc.s0];
  pc.p_last = p.sel_global[pc.s0 + pc.ns - 1];
  const int64_t kb = (int64_t)pc.lo + (int64_t)up.chunk * p.key_chunk;
  if (kb > pc.p_last) return;  // whole chunk after the tile's last row (uniform)
  pc.k_begin = (int)kb;
  pc.k_end = (int)min((int64_t)pc.p_last + 1, kb + p.key_chunk);
  pc.n_active = (int)((pc.p_last - pc.lo) / p.key_chunk) + 1;
  pc.item = up.tbase + pc.tile;
  constexpr int64_t UNIT = partial_bytes<HD, C::QT>();
  const int64_t ustride = (int64_t)up.tr * p.hkv * UNIT;
  pc.own = pc.n_active > 1 ? p.ws + ((int64_t)u * p.hkv + g) * UNIT : nullptr;
  pc.part0 = pc.n_active > 1
                 ? p.ws + ((up.ubase + (int64_t)(up.tr - 1 - pc.tile)) * p.hkv + g) * UNIT
                 : nullptr;
  pc.part1 = pc.n_active > 1 ? pc.part0 + ustride : nullptr;
  pc.part_stride = ustride;
  attn_piece<HD, KS>(p, g, pc, kst, vst, s_last);
}

// Units in their own order: workgroup b runs unit b / hkv of KV head b % hkv
// (within a request chunk by chunk, each chunk from its last query tile to
// its first).
template <int HD, int KS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_mfma_kernel(const AttnParams p) {
  using C = AttnCfg<HD, KS>;
  __shared__ __attribute__((aligned(1024))) bf16 kst[C::STAGES][C::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vst[C::STAGES][C::TILE];
  __shared__ int s_last;
  attn_unit<HD, KS>(p, (int)(blockIdx.x / p.hkv), (int)(blockIdx.x % p.hkv), kst, vst, s_last);
}

// Units in a launch order chosen on the host: workgroup b runs unit
// ord.e[b / hkv] of KV head b % hkv.  The hardware hands out workgroups in
// launch order, so listing the longest pieces first leaves the short ones to
// fill the end of the launch (list scheduling, longest first) instead of
// the last key chunks of the long rows.
template <int HD, int KS, int N>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_ordered_kernel(const AttnParams p, const AttnOrder<N> ord) {
  using C = AttnCfg<HD, KS>;
  __shared__ __attribute__((aligned(1024))) bf16 kst[C::STAGES][C::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vst[C::STAGES][C::TILE];
  __shared__ int s_last;
  attn_unit<HD, KS>(p, (int)ord.e[blockIdx.x / p.hkv], (int)(blockIdx.x % p.hkv), kst, vst,
                    s_last);
}

// The balanced decomposition (p.spans workgroups per KV head, key split 1).
template <int HD>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void attn_stream_kernel(const AttnParams p) {
  using C = AttnCfg<HD, 1>;
  __shared__ __attribute__((aligned(1024))) bf16 kst[C::STAGES][C::TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vst[C::STAGES][C::TILE];
  __shared__ int s_last;
  __shared__ uint32_t tb[kStreamMaxRequests + 1], gt[kStreamMaxTiles + 1], tmp[kWaves];
  __shared__ uint32_t s_maxn;
  attn_stream<HD>(p, (int)(blockIdx.x % p.hkv), kst, vst, s_last, tb, gt, tmp, s_maxn);
}

// Arrival counters of a split launch set to zero before it (standalone calls
// on a workspace of unknown contents; inside cb_blend_layer the fuse launch
// clears them).
__global__ __launch_bounds__(256) void attn_clear_kernel(unsigned *cnt, int32_t n) {
  for (int i = blockIdx.x * 256 + (int)threadIdx.x; i < n; i += gridDim.x * 256) cnt[i] = 0;
}

int attn_mfma_rows_per_tile(int dtype, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int key_split) {
  if (dtype != kBF16) return 0;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return 0;
  if (key_split != 1 && key_split != 2) return 0;
  const int qt = kQT / key_split;
  const int group = n_q_heads / n_kv_heads;
  if (group < 1 || group > qt || qt % group != 0) return 0;
  return qt / group;
}

size_t attn_unit_bytes(int32_t head_dim, int key_split) {
  const size_t qt = (size_t)(kQT / key_split);
  return qt * head_dim * 2 + 3 * qt * sizeof(float);
}

int attn_max_chunks() { return kMaxChunks; }

bool attn_stream_fits(int32_t n_req, int64_t tiles) {
  return n_req <= kStreamMaxRequests && tiles <= kStreamMaxTiles;
}

template <int HD, int KS, int N>
static hipError_t launch_ordered(const AttnParams &p, const dim3 grid, const uint32_t *ord,
                                 int64_t n, hipStream_t stream) {
  AttnOrder<N> o{};  // entries past n are never read; zeroed all the same
  std::copy(ord, ord + n, o.e);
  hipLaunchKernelGGL((attn_ordered_kernel<HD, KS, N>), grid, dim3(64 * kWaves), 0, stream, p, o);
  return hipGetLastError();
}

template <int HD, int KS>
static hipError_t launch_hd(const AttnParams &p, const AttnPlan &plan, int n_kv_heads,
                            const uint32_t *ord, hipStream_t stream) {
  const dim3 grid((unsigned)(plan.units * n_kv_heads)), block(64 * kWaves);
  if (ord) {
    if (plan.units <= 64) return launch_ordered<HD, KS, 64>(p, grid, ord, plan.units, stream);
    if (plan.units <= 256) return launch_ordered<HD, KS, 256>(p, grid, ord, plan.units, stream);
    return launch_ordered<HD, KS, kMaxOrder>(p, grid, ord, plan.units, stream);
  }
  if constexpr (KS == 1) {
    if (plan.spans > 0) {
      hipLaunchKernelGGL((attn_stream_kernel<HD>), grid, block, 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_mfma_kernel<HD, KS>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// Longest-first launch order of a split plan's units, or false where the
// kernel's own order stands: unsplit plans (their units run request by
// request, last tile first, so the workgroups side by side on an XCD share
// one request's K/V rows in its L2 -- ordering them across requests bought
// no time and tripled the L2 misses), the balanced decomposition, and more
// units than the table holds.  A tile's row ends at its last selected row's
// position, which only the device knows; the host estimates it as if
// request r's k_r selected rows were spread evenly over its n_r tokens
// (rows_end * n_r / k_r) and ranks units by the keys of their chunk before
// that end.
static bool attn_launch_order(const AttnArgs &a, const AttnPlan &plan, uint32_t *ord) {
  if (plan.spans > 0 || !plan.split || plan.units > kMaxOrder) return false;
  if (!a.h_tok_off || !a.h_sel_off) return false;
  struct Item { int64_t keys; uint32_t u; };
  Item items[kMaxOrder];
  int64_t n = 0, ubase = 0;
  const int rows = plan.rows_per_tile;
  const int64_t kc = plan.key_chunk;
  for (int32_t r = 0; r < a.n_req; ++r) {
    const int64_t kr = (int64_t)a.h_sel_off[r + 1] - a.h_sel_off[r];
    const int64_t nr = (int64_t)a.h_tok_off[r + 1] - a.h_tok_off[r];
    const int64_t tr = (kr + rows - 1) / rows;
    const int64_t cr = (nr + kc - 1) / kc;
    if (n + tr * cr > kMaxOrder) return false;
    for (int64_t c = 0; c < cr; ++c)
      for (int64_t t = 0; t < tr; ++t) {
        const int64_t end = (std::min<int64_t>(kr, (t + 1) * rows) * nr + kr - 1) / kr;
        const int64_t keys = std::max<int64_t>(0, std::min(end, (c + 1) * kc) - c * kc);
        items[n++] = {keys, (uint32_t)(ubase + c * tr + (tr - 1 - t))};
      }
    ubase += tr * cr;
  }
  if (n != plan.units) return false;
  if (!ord) return true;
  std::sort(items, items + n, [](const Item &x, const Item &y) {
    return x.keys != y.keys ? x.keys > y.keys : x.u < y.u;
  });
  for (int64_t i = 0; i < n; ++i) ord[i] = items[i].u;
  return true;
}

hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &plan, bool counters_zero,
                            hipStream_t stream) {
  if (plan.units == 0) return hipSuccess;
  AttnParams p;
  p.out = (bf16 *)a.out;
  p.q_c = (const bf16 *)a.q_c;
  p.sel_local = a.sel_local;
  p.sel_global = a.sel_global;
  p.k_fused = (const bf16 *)a.k_fused;
  p.v_fused = (const bf16 *)a.v_fused;
  p.tok_off = a.tok_off;
  p.sel_off = a.sel_off;
  p.ws = (unsigned char *)a.workspace;
  p.cnt = plan.split ? (unsigned *)((char *)a.workspace + plan.cnt_offset) : nullptr;
  p.n_req = a.n_req;
  p.hq = a.n_q_heads;
  p.hkv = a.n_kv_heads;
  p.group = a.n_q_heads / a.n_kv_heads;
  p.rows_per_tile = plan.rows_per_tile;
  p.key_chunk = plan.key_chunk;
  p.spans = plan.spans;
  p.scale_log2 = a.softmax_scale * 1.4426950408889634f;
  if (plan.key_chunk % (kKeyTile * plan.key_split) != 0) return hipErrorInvalidValue;
  if (plan.spans > 0 && (plan.key_split != 1 || a.n_req > kStreamMaxRequests ||
                         plan.tiles > kStreamMaxTiles))
    return hipErrorInvalidValue;
  if (plan.split && !counters_zero) {
    const int blocks = (int)std::min<int64_t>((plan.n_cnt + 255) / 256, 64);
    hipLaunchKernelGGL(attn_clear_kernel, dim3(blocks), dim3(256), 0, stream, p.cnt,
                       (int32_t)plan.n_cnt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int h = a.n_kv_heads;
  uint32_t order[kMaxOrder];  // on the stack: the library keeps no state between calls
  const uint32_t *ord = attn_launch_order(a, plan, order) ? order : nullptr;
  if (plan.key_split == 2) {
    switch (a.head_dim) {
      case 32: return launch_hd<32, 2>(p, plan, h, ord, stream);
      case 64: return launch_hd<64, 2>(p, plan, h, ord, stream);
      default: return launch_hd<128, 2>(p, plan, h, ord, stream);
    }
  }
  switch (a.head_dim) {
    case 32: return launch_hd<32, 1>(p, plan, h, ord, stream);
    case 64: return launch_hd<64, 1>(p, plan, h, ord, stream);
    default: return launch_hd<128, 1>(p, plan, h, ord, stream);
  }
}

// ---------------------------------------------------------------------------
// Plain kernel for every other geometry (fp32 storage, head_dim 16, group
// sizes that do not divide the MFMA tile): one wave per (selected row, query
// head), 64 keys per step (one per lane), online softmax, fp32 throughout.
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
    if (u <= hi) {  // this lane's key row in 16-byte pieces (head_dim is a multiple of 8)
      const T *kr = k_fused + ((int64_t)u * hkv + g) * hd;
      constexpr int VN = Vec16<T>::N;
      float dot = 0.f;
      for (int d0 = 0; d0 < hd; d0 += VN) {
        float kv[VN];
        Vec16<T>::load(kr + d0, kv);
#pragma unroll
        for (int i = 0; i < VN; ++i) dot = fmaf(qs[d0 + i], kv[i], dot);
      }
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
    // O += P V over this step's keys, eight V rows loaded before their products
    const int nk = min(64, hi - u0 + 1);
    const T *vb = v_fused + ((int64_t)u0 * hkv + g) * hd;
    const int64_t vstride = (int64_t)hkv * hd;
    int kk = 0;
    for (; kk + 8 <= nk; kk += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const T *vr = vb + (kk + j) * vstride;
        v0[j] = lane < hd ? ld(vr + lane) : 0.f;
        v1[j] = lane + 64 < hd ? ld(vr + lane + 64) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc0 = fmaf(ps[kk + j], v0[j], acc0);
        acc1 = fmaf(ps[kk + j], v1[j], acc1);
      }
    }
    for (; kk < nk; ++kk) {
      const T *vr = vb + kk * vstride;
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

// Device helpers shared by the gfx950 kernels of libcacheblend.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cb {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Relaxed accesses at agent scope: performed at the coherence point that
// all XCDs share, so a workgroup on another XCD of the same launch sees them
// (the XCDs' L2 caches are not coherent with each other).
template <typename T> __device__ inline void store_agent(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T> __device__ inline T load_agent(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt operand that waits until at most n vector-memory operations of
// the wave are outstanding (loads, stores and copies to LDS; gfx9 encoding,
// the other counters left alone).
__device__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// s_waitcnt operand for lgkmcnt(0) with the VM counter left free (gfx9
// encoding; vmcnt(n) is waitcnt_vm).
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Workgroup barrier after which every wave's LDS accesses before it are
// complete; neither the compiler nor the scheduler moves work across it.
// Global loads, and copies into LDS, stay in flight: their completion is
// waited for where their data is used (__syncthreads waits for them too).
__device__ inline void phase_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte vector of storage elements, converted to/from fp32.
template <typename T> struct Vec16;

template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static inline void load(const float *p, float (&x)[4]) {
    float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static inline void store(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ static inline void load(const bf16 *p, float (&x)[8]) {
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  // Round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
  __device__ static inline void store(bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
    *reinterpret_cast<bf16x8 *>(p) = v;
  }
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

}  // namespace cb

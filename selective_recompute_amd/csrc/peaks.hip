// Attainable peaks of one MI355X, measured rather than quoted: dense bf16
// MFMA throughput of v_mfma_f32_32x32x16_bf16 (the instruction the attention
// uses) with independent accumulators, on slowly varying and on
// pseudo-random operands, and the HBM bandwidth of a plain
// 16-byte copy and of a streaming read over buffers far larger than the
// 256 MB Infinity Cache.  Prints one JSON object on stdout.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                            \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

constexpr int kAcc = 8;  // independent accumulators per wave
constexpr int kOps = 4;  // distinct A and B operands per wave

// Value in [-1, 1) from a 32-bit integer hash (splitmix-style finaliser).
__device__ inline float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

// SMOOTH = 1: slowly varying operands (few bits toggle between MFMAs);
// SMOOTH = 0: pseudo-random operands, rotated every product like the K/V
// fragments of the attention -- the rate that real data sees, since the
// chip lowers its clock when more bits toggle.
template <int SMOOTH>
__global__ __launch_bounds__(256) void mfma_loop(float *sink, int iters) {
  bf16x8 a[kOps], b[kOps];
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int o = 0; o < kOps; ++o)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[o][i] = SMOOTH ? (__bf16)(0.001f * (float)(threadIdx.x + i))
                       : (__bf16)hash_unit(t * 64u + (uint32_t)(o * 8 + i));
      b[o][i] = SMOOTH ? (__bf16)(0.002f * (float)i)
                       : (__bf16)hash_unit(t * 64u + 32u + (uint32_t)(o * 8 + i));
    }
  f32x16 c[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j % kOps], b[(j / 2) % kOps], c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += c[j][0];
  if (s == 1234.5f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;  // never true: keeps the work
}

__global__ __launch_bounds__(256) void copy16(uint4 *__restrict__ dst, const uint4 *__restrict__ src,
                                              size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read16(const uint4 *__restrict__ src, size_t n, uint32_t *sink) {
  uint32_t x = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (x == 0x12345678u) sink[0] = x;  // practically never: keeps the loads
}

template <typename F>
static float best_ms(F launch, int reps) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();  // warm-up
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int r = 0; r < reps; ++r) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  CHECK(hipGetLastError());
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;

  // MFMA: 4 workgroups of 4 waves per CU, 8 accumulators per wave.
  float *sink;
  const int mblocks = cus * 4, iters = 4096;
  CHECK(hipMalloc(&sink, (size_t)mblocks * 256 * sizeof(float)));
  const float mfma_ms = best_ms([&] {
    hipLaunchKernelGGL(mfma_loop<1>, dim3(mblocks), dim3(256), 0, 0, sink, iters);
  }, 3);
  const float mfma_rnd_ms = best_ms([&] {
    hipLaunchKernelGGL(mfma_loop<0>, dim3(mblocks), dim3(256), 0, 0, sink, iters);
  }, 3);
  const double mfma_flops = (double)mblocks * 4 * iters * kAcc * (2.0 * 32 * 32 * 16);

  // HBM: 2 GiB buffers.
  const size_t bytes = (size_t)2 << 30, n = bytes / 16;
  uint4 *a, *b;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMemset(a, 1, bytes));
  CHECK(hipMemset(b, 2, bytes));
  const int sblocks = cus * 16;
  const float copy_ms = best_ms([&] {
    hipLaunchKernelGGL(copy16, dim3(sblocks), dim3(256), 0, 0, b, a, n);
  }, 5);
  const float read_ms = best_ms([&] {
    hipLaunchKernelGGL(read16, dim3(sblocks), dim3(256), 0, 0, a, n, (uint32_t *)sink);
  }, 5);
  printf("{\"device\": \"%s\", \"cus\": %d, \"mfma_bf16_32x32x16_tflops\": %.1f, "
         "\"mfma_bf16_32x32x16_random_tflops\": %.1f, \"copy_gbs\": %.1f, \"read_gbs\": %.1f}\n",
         prop.gcnArchName, cus, mfma_flops / (mfma_ms * 1e-3) / 1e12,
         mfma_flops / (mfma_rnd_ms * 1e-3) / 1e12,
         2.0 * bytes / (copy_ms * 1e-3) / 1e9, (double)bytes / (read_ms * 1e-3) / 1e9);
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(sink));
  return 0;
}

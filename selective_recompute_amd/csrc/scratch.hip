// Device scratch that the library owns, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the attention's split partials and arrival counters of
// cb_blend_layer_noalloc live here instead of in a caller's workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, from the code object's load
// until the process ends.  In host code its name is only a stand-in, not a
// device address; the address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept per device.
#include <mutex>

#include "cb_launch.hpp"

namespace cb {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace cb

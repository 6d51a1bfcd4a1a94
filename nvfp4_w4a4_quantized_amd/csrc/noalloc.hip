// The library's one fixed device workspace, for callers that cannot allocate.
//
// nvfp4_w4a4_linear_noalloc runs the whole layer like nvfp4_w4a4_linear, but the
// shapes that run in two stages keep the quantized activations (codes, then scale
// bytes) here instead of in caller-provided buffers.  Each GPU the library runs on
// holds its own copy of the array until the process ends.  Calls that overlap on
// one GPU share it and race; every call overwrites all the bytes it reads, so
// nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace nvfp4 {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];        // per device: the array's device address
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // with this device current: the address of this device's copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace nvfp4

// noalloc.hip -- the library's own fixed scratch, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array. Each GPU the library runs on holds its own copy
// from the module's load until the process ends, at its own address; the host-side name of
// the array is only a registration handle, so kernels are given the device address that
// hipGetSymbolAddress returns, looked up once per device (with that device current) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[mamba::kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace mamba {

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mamba

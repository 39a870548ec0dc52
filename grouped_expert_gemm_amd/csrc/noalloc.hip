// Library-held scratch for the entry point that allocates nothing
// (gnf4_grouped_gemm_noalloc): one static device array per GPU, holding what a
// caller's workspace holds for gnf4_grouped_gemm (split-K counters and partials,
// the row-scaled fp16 activations and their row exponents).
//
// In host code the array's name is a host-side stand-in, not a device address.
// Its device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "geg_launch.hpp"

namespace geg {

namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // The header's error word starts at zero. A fill kernel, not a memset, so
    // that a first call under graph capture records a plain kernel node.
    e = launch_zero(p, kNoallocZeroBytes, stream);
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace geg

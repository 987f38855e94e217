// Static device scratch of the allocation-free entry point
// (nvfp4_quantize_gemm_no_alloc): the quantized activations of a
// quantize + GEMM call go here instead of a caller-provided workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds one copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol: the device address
// is looked up once per device with hipGetSymbolAddress and kept, and only
// that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t no_alloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nvfp4

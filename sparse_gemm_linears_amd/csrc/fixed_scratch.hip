// The library's fixed scratch array: device memory that exists from the moment
// the code object is loaded on a device until the process ends, for callers
// that cannot allocate (code under HIP graph capture that must not add memory
// nodes, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array.  Its name in host code is only the
// host-side handle of the symbol, not a device address: the address of each
// device's copy comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace fp8lin {
namespace {

// Enough for every split-K plan on a 256-CU device: K is split only when the
// tiles are 128 tokens high and cover at most half of the compute units, with
// at most one split workgroup per compute unit, each holding one fp32 tile of
// 128 x 256 (256 x 128 KiB); the weight-streaming kernel's splits need at most
// 4 x 32 tokens x 6143 rows.
constexpr size_t kFixedScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kFixedScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t fixed_scratch(void **p, size_t *bytes) {
  *p = nullptr;
  *bytes = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
  }
  *p = g_ptr[dev];
  *bytes = kFixedScratchBytes;
  return hipSuccess;
}

}  // namespace fp8lin

// The workspace of moe_forward_noalloc: a fixed device array, so that entry point allocates
// nothing (for callers that cannot call hipMalloc: code under HIP graph capture, serving loops,
// harnesses that forbid allocation). Each GPU the library runs on holds its own copy of the array
// from the time the library's code is loaded on it until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address: host code reaches the
// array only through scratch_address(), which asks the runtime for this device's copy once per
// device (with that device current) and keeps the answer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace moe {

namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_address(void **ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe

// Static device scratch of moe_forward_noalloc: the workspace of the layer's
// forward for callers that cannot allocate device memory.
//
// One file-scope array per GPU the library runs on (the code object's global is
// instantiated on every device it is loaded on, and held until the process
// ends).  In host code `scratch` names a host-side stand-in, not device memory,
// so it is never passed to a kernel or a copy: the first call on a device, with
// that device current, asks the runtime for the array's device address on that
// device and caches it; every later call on that device uses the cached address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe

// Library-held scratch memory for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops that must not call the allocator, harnesses that forbid it).
//
// One file-scope device array per GPU, kScratchBytes long, lives as long as the process. Host
// code never passes the array's name to a kernel (on the host it names a stand-in, not device
// memory): the first use on a device looks its device address up with hipGetSymbolAddress,
// with that device current, and every later use on that device takes the cached address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace rlt {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_region(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace rlt

// Split scratch for callers that cannot allocate (graph capture, serving
// loops, harnesses that forbid hipMalloc): one file-scope device array per
// GPU, whose device address is looked up once per device with that device
// current.  Host code uses only the looked-up address, never the array's
// name (which in host code is a stand-in, not a device address).
#include <mutex>

#include "mlasd_internal.h"

namespace mlasd {

// 16 MiB holds the fp32 partials of every automatically planned split up to
// B = 56 at top-k 512 on 256 CUs (the largest, B = 56 at 2 slices, needs
// 12.9 MB).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};
}  // namespace

hipError_t noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mlasd

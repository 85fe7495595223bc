// Fixed device scratch of the no-allocation forward entry point (for callers that cannot
// call hipMalloc: code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The array lives in the library's code object, so every device the library
// runs on holds its own copy of SFFN_NOALLOC_SCRATCH_BYTES until the process ends.  Host
// code never uses the array's name as a device address: the address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept per device.
#include <mutex>

#include "sffn_common.hpp"

namespace sffn {

static __device__ __align__(256) unsigned char scratch[SFFN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return e;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sffn

// Static device scratch for the allocation-free entry points (callers that cannot allocate:
// code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array of kStaticScratchBytes; every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in symbol): the first call on a device, with that
// device current, looks up the array's device address with hipGetSymbolAddress and keeps it
// per device; kernels receive that address.  Every call on one GPU shares the array and it
// keeps the last call's contents, so calls that overlap in time on one GPU race.
#include <mutex>

#include "pf_internal.h"

namespace pf {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pf

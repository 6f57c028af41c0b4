// Fixed device scratch of the no-allocation forward (lb_linear_forward_noalloc
// in include/littlebit.h): a file-scope device array of kNoAllocScratchBytes,
// one copy per GPU (each device that loads this library holds it until the
// process ends).  Host code never passes the array's name to a kernel: it is
// a host-side stand-in, not a device address.  The address each device gives
// the array is looked up once per device, with that device current, and kept.
#include <mutex>

#include "lb_internal.h"

static __device__ __align__(256) unsigned char scratch[lb::kNoAllocScratchBytes];

namespace lb {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the lookup must run with `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace lb

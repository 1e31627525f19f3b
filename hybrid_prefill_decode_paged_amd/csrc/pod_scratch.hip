// Device scratch of pod_attn_run_noalloc: one fixed array per GPU that stands in for the caller's
// workspace, for callers that cannot allocate device memory.  The array lives in this file's
// code object; its device address is looked up once per device (with that device current) and
// kept, and only that address is ever handed to kernels or copies: in host code the array's name
// is a host-side stand-in, not a device address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[pod::kNoAllocScratchBytes];

namespace pod {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;       // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace pod

// Device scratch of the allocation-free fused entry point (pdssm_fwd_noalloc):
// the look-back workspace of one call lives in a file-scope device array
// instead of caller memory.  Each GPU holds its own copy of the array, at its
// own address, for the life of the process; every call on that GPU shares it.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: the address a kernel may use is resolved once per device with
// hipGetSymbolAddress (with that device current) and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pdscan_plan.h"

namespace pdscan {

constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;   // must match PDSSM_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of the current device's scratch array and its size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kNoallocScratchBytes;
  return hipSuccess;
}

}  // namespace pdscan

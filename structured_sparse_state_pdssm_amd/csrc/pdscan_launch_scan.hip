// Launcher for the scan mode (selections given), and the workspace clear
// that precedes every scan or fused launch.
#include "pdscan_device.h"

namespace pdscan {

// Zero the workspace words the look-back reads (header, aggregates,
// inclusive states): every word starts untagged.
__global__ void clear_kernel(uint64_t* w, size_t n) {
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    w[q] = 0;
}

void launch_clear(const Args& a, hipStream_t st) {
  const size_t words = a.p.ws_bytes / 8;
  size_t cb = (words + 255) / 256;
  if (cb > 4096) cb = 4096;
  if (cb < 1) cb = 1;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)cb), dim3(256), 0, st, (uint64_t*)a.ws, words);
}

// status[0] |= the error word of the call that last used the workspace
__global__ void status_kernel(const uint32_t* hdr, uint32_t* status) {
  if (threadIdx.x == 0)
    status[0] |= __hip_atomic_load(hdr + kWsError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_status(const void* ws, uint32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(status_kernel, dim3(1), dim3(64), 0, st, (const uint32_t*)ws, status);
  return hipGetLastError();
}

hipError_t launch_scan(const Args& a, hipStream_t st) {
  launch_clear(a, st);
  if (a.p.step16) {
    if (a.H_all)
      hipLaunchKernelGGL((pdssm_step16_kernel<0, 1, 1>), dim3(a.p.tasks), dim3(kThreads), a.p.lds_bytes, st, a);
    else if (a.p.n_out > 1)
      hipLaunchKernelGGL((pdssm_step16_kernel<0, kMaxOut>), dim3(a.p.tasks), dim3(kThreads), a.p.lds_bytes, st, a);
    else if (a.P_in)
      hipLaunchKernelGGL(pdssm_step16_kernel<1>, dim3(a.p.tasks), dim3(kThreads), a.p.lds_bytes, st, a);
    else
      hipLaunchKernelGGL(pdssm_step16_kernel<0>, dim3(a.p.tasks), dim3(kThreads), a.p.lds_bytes, st, a);
    return hipGetLastError();
  }
  if (a.p.n_out > 1) {                             // several rows of C (general scan)
    switch (npt_of(a.p)) {
      case 32: launch_kernel<kModeScan, 0, 0, kSelAny, 32, false, kMaxOut>(a, st); break;
      case 64: launch_kernel<kModeScan, 0, 0, kSelAny, 64, false, kMaxOut>(a, st); break;
      default: launch_kernel<kModeScan, 0, 0, kSelAny, 0, false, kMaxOut>(a, st); break;
    }
    return hipGetLastError();
  }
  switch (npt_of(a.p)) {
    case 8: launch_kernel<kModeScan, 0, 0, kSelAny, 8, false>(a, st); break;
    case 16: launch_kernel<kModeScan, 0, 0, kSelAny, 16, false>(a, st); break;
    case 32: launch_kernel<kModeScan, 0, 0, kSelAny, 32, false>(a, st); break;
    case 64: launch_kernel<kModeScan, 0, 0, kSelAny, 64, false>(a, st); break;
    default: launch_kernel<kModeScan, 0, 0, kSelAny, 0, false>(a, st); break;
  }
  return hipGetLastError();
}

}  // namespace pdscan

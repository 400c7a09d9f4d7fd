// Launcher of the gradient pass through the scan: workspace clear, the
// backward kernel, and the ordered reduction of the dC partials.
#include "pdscan_bwd.h"

namespace pdscan {

__global__ void bwd_clear_kernel(uint64_t* w, size_t n) {
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    w[q] = 0;
}

hipError_t launch_bwd(const BwdArgs& a, float* g_C, hipStream_t st) {
  const Plan& p = a.p;
  const size_t words = p.ws_bytes / 8;             // header, maps and carries
  size_t cb = (words + 255) / 256;
  if (cb > 4096) cb = 4096;
  if (cb < 1) cb = 1;
  hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)cb), dim3(256), 0, st, (uint64_t*)a.ws, words);
  if (p.N <= 16)
    hipLaunchKernelGGL(pdssm_bwd_kernel<true>, dim3((unsigned)p.tasks), dim3(kThreads), (unsigned)a.l.bytes, st, a);
  else
    hipLaunchKernelGGL(pdssm_bwd_kernel<false>, dim3((unsigned)p.tasks), dim3(kThreads), (unsigned)a.l.bytes, st, a);
  hipLaunchKernelGGL(pdssm_bwd_reduce_c, dim3((unsigned)p.H), dim3(kThreads), 0, st,
                     (const float*)(a.ws + a.ws_gc), g_C, p.nC, p.B, p.H, p.N);
  return hipGetLastError();
}

}  // namespace pdscan

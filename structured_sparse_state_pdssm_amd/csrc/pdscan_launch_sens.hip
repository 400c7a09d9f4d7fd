// Launcher of the impulse-sensitivity pass: workspace clear, then the
// chunked kernel.
#include "pdscan_sens.h"

namespace pdscan {

__global__ void sens_clear_kernel(uint64_t* w, size_t n) {
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    w[q] = 0;
}

hipError_t launch_sens(const SensArgs& a, hipStream_t st) {
  const SensPlan& q = a.q;
  const size_t words = q.ws_bytes / 8;
  size_t cb = (words + 255) / 256;
  if (cb > 8192) cb = 8192;
  if (cb < 1) cb = 1;
  hipLaunchKernelGGL(sens_clear_kernel, dim3((unsigned)cb), dim3(256), 0, st, (uint64_t*)a.ws, words);
  const dim3 grid((unsigned)q.tasks), block(kThreads);
  switch (q.d / 16) {
    case 1: hipLaunchKernelGGL(pdssm_sens_kernel<1>, grid, block, (unsigned)q.bytes, st, a); break;
    case 2: hipLaunchKernelGGL(pdssm_sens_kernel<2>, grid, block, (unsigned)q.bytes, st, a); break;
    case 3: hipLaunchKernelGGL(pdssm_sens_kernel<3>, grid, block, (unsigned)q.bytes, st, a); break;
    case 4: hipLaunchKernelGGL(pdssm_sens_kernel<4>, grid, block, (unsigned)q.bytes, st, a); break;
    case 5: hipLaunchKernelGGL(pdssm_sens_kernel<5>, grid, block, (unsigned)q.bytes, st, a); break;
    case 6: hipLaunchKernelGGL(pdssm_sens_kernel<6>, grid, block, (unsigned)q.bytes, st, a); break;
    case 7: hipLaunchKernelGGL(pdssm_sens_kernel<7>, grid, block, (unsigned)q.bytes, st, a); break;
    default: hipLaunchKernelGGL(pdssm_sens_kernel<8>, grid, block, (unsigned)q.bytes, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace pdscan

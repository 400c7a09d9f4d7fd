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
  hipLaunchKernelGGL(pdssm_sens_kernel, dim3((unsigned)q.tasks), dim3(kThreads), (unsigned)q.bytes, st, a);
  return hipGetLastError();
}

}  // namespace pdscan

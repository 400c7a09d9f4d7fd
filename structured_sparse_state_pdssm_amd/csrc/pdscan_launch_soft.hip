// Launcher of the soft-selection comparison pass.
#include "pdscan_soft.h"

namespace pdscan {

hipError_t launch_soft(const SoftArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.q.tasks), block(kThreads);
  const unsigned lds = (unsigned)a.q.bytes;
  switch (a.q.d) {
    case 16: hipLaunchKernelGGL(pdssm_soft_kernel<4>, grid, block, lds, st, a); break;
    case 32: hipLaunchKernelGGL(pdssm_soft_kernel<8>, grid, block, lds, st, a); break;
    case 64: hipLaunchKernelGGL(pdssm_soft_kernel<16>, grid, block, lds, st, a); break;
    case 128: hipLaunchKernelGGL(pdssm_soft_kernel<32>, grid, block, lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dict_hardmax(const float* M, int32_t* dict, int HK, int N, hipStream_t st) {
  const int n = HK * N;
  hipLaunchKernelGGL(pdssm_dict_hardmax_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, M, dict, HK, N);
  return hipGetLastError();
}

}  // namespace pdscan

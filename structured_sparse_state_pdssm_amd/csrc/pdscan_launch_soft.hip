// Launcher of the soft-selection comparison pass.
#include "pdscan_soft.h"

namespace pdscan {

hipError_t launch_soft(const SoftArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pdssm_soft_kernel, dim3((unsigned)a.q.tasks), dim3(kThreads), (unsigned)a.q.bytes, st, a);
  return hipGetLastError();
}

hipError_t launch_dict_hardmax(const float* M, int32_t* dict, int HK, int N, hipStream_t st) {
  const int n = HK * N;
  hipLaunchKernelGGL(pdssm_dict_hardmax_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, M, dict, HK, N);
  return hipGetLastError();
}

}  // namespace pdscan

// Launcher for the fused selection + scan on the step-major kernels (per-head
// u, N <= 16, K <= 16): the impulse and base shapes.  The general kernel's
// launcher is in its own unit (compiled in parallel).
#include "pdscan_device.h"

namespace pdscan {

void launch_clear(const Args& a, hipStream_t st);

hipError_t launch_fused16(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  launch_clear(a, st);
  if (p.fused16 && p.fold_bu && p.n_out == 2) {
    const dim3 grid(p.tasks), block(kThreads);
    if (p.in_bf16)
      hipLaunchKernelGGL((pdssm_fused16_kernel<1, 1, 4, 0, 1, 2>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 64)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 4, 1, 1, 2>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 32)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 2, 1, 1, 2>), grid, block, p.lds_bytes, st, a);
    else
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 1, 0, 1, 2>), grid, block, p.lds_bytes, st, a);
    return hipGetLastError();
  }
  if (p.fused16 && p.fold_bu && p.n_out > 1) {
    const dim3 grid(p.tasks), block(kThreads);
    if (p.in_bf16)
      hipLaunchKernelGGL((pdssm_fused16_kernel<1, 1, 4, 0, 1, kMaxOut>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 64)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 4, 1, 1, kMaxOut>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 32)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 2, 1, 1, kMaxOut>), grid, block, p.lds_bytes, st, a);
    else
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 1, 0, 1, kMaxOut>), grid, block, p.lds_bytes, st, a);
    return hipGetLastError();
  }
  if (p.fused16 && p.fold_bu) {
    const dim3 grid(p.tasks), block(kThreads);
    if (p.in_bf16)
      hipLaunchKernelGGL((pdssm_fused16_kernel<1, 1, 4, 0, 1>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 64)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 4, 1, 1>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 32)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 2, 1, 1>), grid, block, p.lds_bytes, st, a);
    else
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 1, 0, 1>), grid, block, p.lds_bytes, st, a);
    return hipGetLastError();
  }
  if (p.fused16) {
    const dim3 grid(p.tasks), block(kThreads);
    if (p.in_bf16)
      hipLaunchKernelGGL((pdssm_fused16_kernel<1, 1, 4, 0>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 64)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 4, 1>), grid, block, p.lds_bytes, st, a);
    else if (p.d == 32)
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 2, 1>), grid, block, p.lds_bytes, st, a);
    else
      hipLaunchKernelGGL((pdssm_fused16_kernel<0, 0, 1, 0>), grid, block, p.lds_bytes, st, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;   // not a step-major plan
}

}  // namespace pdscan

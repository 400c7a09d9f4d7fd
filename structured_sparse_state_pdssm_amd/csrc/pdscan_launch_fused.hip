// Launcher for the fused selection + scan (the hot path): the step-major
// kernels (own unit), or the general kernel with one row of C (here) or
// several (own unit).
#include "pdscan_launch_general.h"

namespace pdscan {

void launch_clear(const Args& a, hipStream_t st);
hipError_t launch_fused16(const Args& a, hipStream_t st);       // pdscan_launch_fused16.hip
hipError_t launch_general_multi(const Args& a, hipStream_t st);  // pdscan_launch_fused_multi.hip
hipError_t launch_general_fold(const Args& a, hipStream_t st);   // pdscan_launch_fused_fold.hip

hipError_t launch_fused(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  if (p.fused16) return launch_fused16(a, st);
  launch_clear(a, st);
  // several outputs come only with the drive folded (pdssm_fwd_wb_multi)
  if (p.n_out > 1) return launch_general_multi(a, st);
  return p.fold_bu ? launch_general_fold(a, st) : launch_general<1, 0>(a, st);
}

}  // namespace pdscan

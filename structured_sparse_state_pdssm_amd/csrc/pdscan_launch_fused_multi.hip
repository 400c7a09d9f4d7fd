// Launcher for the general kernel's fused pass with several rows of C per
// head (pdssm_fwd_wb_multi off the step-major kernels: the drive is folded).
#include "pdscan_launch_general.h"

namespace pdscan {

hipError_t launch_general_multi(const Args& a, hipStream_t st) { return launch_general<kMaxOut, 1>(a, st); }

}  // namespace pdscan

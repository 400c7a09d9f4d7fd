// Launcher for the general kernel's fused pass with the drive folded into the
// selection GEMM (pdssm_fwd_wb off the step-major kernels).
#include "pdscan_launch_general.h"

namespace pdscan {

hipError_t launch_general_fold(const Args& a, hipStream_t st) { return launch_general<1, 1>(a, st); }

}  // namespace pdscan

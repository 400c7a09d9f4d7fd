// Launcher for the selection-only mode (scores, argmax, logistic).
#include "pdscan_device.h"

namespace pdscan {

hipError_t launch_select(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  const int path = sel_path(p);
  if (p.in_bf16 && p.mma_bf16) {
    if (path == kSelBF16D128N3) launch_kernel<kModeSelect, 1, 1, kSelBF16D128N3, 0, true>(a, st);
    else if (path == kSelDeep + 2) launch_kernel<kModeSelect, 1, 1, kSelDeep + 2, 0, true>(a, st);
    else if (path == kSelDeep + 4) launch_kernel<kModeSelect, 1, 1, kSelDeep + 4, 0, true>(a, st);
    else if (path == kSelDeep + 6) launch_kernel<kModeSelect, 1, 1, kSelDeep + 6, 0, true>(a, st);
    else if (path > kSelDeep) launch_kernel<kModeSelect, 1, 1, kSelDeep + 8, 0, true>(a, st);
    else launch_kernel<kModeSelect, 1, 1, kSelAny, 0, true>(a, st);
  } else if (p.in_bf16) {
    launch_kernel<kModeSelect, 1, 0, kSelAny, 0, true>(a, st);
  } else if (path == kSelF32D64N2) {
    launch_kernel<kModeSelect, 0, 0, kSelF32D64N2, 0, false>(a, st);
  } else if (path == kSelF32D16N1) {
    launch_kernel<kModeSelect, 0, 0, kSelF32D16N1, 0, false>(a, st);
  } else {
    launch_kernel<kModeSelect, 0, 0, kSelAny, 0, true>(a, st);
  }
  return hipGetLastError();
}

}  // namespace pdscan

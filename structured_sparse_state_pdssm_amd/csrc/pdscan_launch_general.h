// The general kernel's fused-pass launches (every shape outside the
// step-major kernels), templated on the number of rows of C an instantiation
// handles (NOUT = 1, or kMaxOut for the multi-output plans) and on whether
// the drive is folded (FOLD): one instantiation set per launcher unit
// (pdscan_launch_fused.hip: plain; pdscan_launch_fused_fold.hip: folded;
// pdscan_launch_fused_multi.hip: folded, several outputs), compiled in
// parallel.  Only the shape classes that have a specialised selection path
// get a compile-time group width.
#pragma once

#include "pdscan_device.h"

namespace pdscan {

template <int MODE, int NCT, int NOUT, int FOLD>
static void launch_deep_n(const Args& a, hipStream_t st, int npt) {
  if (npt == 64) launch_kernel<MODE, 1, 1, kSelDeep + NCT, 64, true, NOUT, FOLD>(a, st);
  else launch_kernel<MODE, 1, 1, kSelDeep + NCT, 0, true, NOUT, FOLD>(a, st);
}
template <int MODE, int NOUT, int FOLD>
static void launch_deep(const Args& a, hipStream_t st, int nct, int npt) {
  switch (nct) {
    case 2: launch_deep_n<MODE, 2, NOUT, FOLD>(a, st, npt); break;
    case 4: launch_deep_n<MODE, 4, NOUT, FOLD>(a, st, npt); break;
    case 6: launch_deep_n<MODE, 6, NOUT, FOLD>(a, st, npt); break;
    case 8: launch_deep_n<MODE, 8, NOUT, FOLD>(a, st, npt); break;
    default: launch_deep_n<MODE, kFoldMaxTiles, NOUT, FOLD>(a, st, npt); break;   // drive folded
  }
}

template <int NOUT, int FOLD>
static hipError_t launch_general(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  const int path = sel_path(p), npt = npt_of(p);
  if (p.in_bf16 && p.mma_bf16) {
    if (path == kSelStep32) {                      // step-major selection tiles (one output, unfolded)
      if constexpr (NOUT == 1 && !FOLD) launch_kernel<kModeFused, 1, 1, kSelStep32, 32, true, 1, 0>(a, st);
    } else if (path == kSelBF16D128N3 && npt == 32)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N3, 32, true, NOUT, FOLD>(a, st);
    else if (path == kSelBF16D128N3)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N3, 0, true, NOUT, FOLD>(a, st);
    else if (path == kSelBF16D128N5 && npt == 32)            // drive folded, N = 32
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N5, 32, true, NOUT, FOLD>(a, st);
    else if (path == kSelBF16D128N5)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N5, 0, true, NOUT, FOLD>(a, st);
    else if (path > kSelDeep)
      launch_deep<kModeFused, NOUT, FOLD>(a, st, path - kSelDeep, npt);
    else if (npt == 64)
      launch_kernel<kModeFused, 1, 1, kSelAny, 64, true, NOUT, FOLD>(a, st);
    else
      launch_kernel<kModeFused, 1, 1, kSelAny, 0, true, NOUT, FOLD>(a, st);
  } else if (p.in_bf16) {
    launch_kernel<kModeFused, 1, 0, kSelAny, 0, true, NOUT, FOLD>(a, st);
  } else if (path == kSelF32D64N2) {
    if (npt == 16) launch_kernel<kModeFused, 0, 0, kSelF32D64N2, 16, false, NOUT, FOLD>(a, st);
    else launch_kernel<kModeFused, 0, 0, kSelF32D64N2, 0, false, NOUT, FOLD>(a, st);
  } else if (path == kSelF32D16N1) {
    if (npt == 8) launch_kernel<kModeFused, 0, 0, kSelF32D16N1, 8, false, NOUT, FOLD>(a, st);
    else launch_kernel<kModeFused, 0, 0, kSelF32D16N1, 0, false, NOUT, FOLD>(a, st);
  } else {
    launch_kernel<kModeFused, 0, 0, kSelAny, 0, true, NOUT, FOLD>(a, st);
  }
  return hipGetLastError();
}

}  // namespace pdscan

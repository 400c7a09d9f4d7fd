// Launcher for the fused selection + scan (the hot path).  Only the shape
// classes that have a specialised selection path get a compile-time group
// width; everything else runs the general body.
#include "pdscan_device.h"

namespace pdscan {

void launch_clear(const Args& a, hipStream_t st);

template <int MODE, int NCT>
static void launch_deep_n(const Args& a, hipStream_t st, int npt) {
  if (npt == 64) launch_kernel<MODE, 1, 1, kSelDeep + NCT, 64, true>(a, st);
  else launch_kernel<MODE, 1, 1, kSelDeep + NCT, 0, true>(a, st);
}
template <int MODE>
static void launch_deep(const Args& a, hipStream_t st, int nct, int npt) {
  switch (nct) {
    case 2: launch_deep_n<MODE, 2>(a, st, npt); break;
    case 4: launch_deep_n<MODE, 4>(a, st, npt); break;
    case 6: launch_deep_n<MODE, 6>(a, st, npt); break;
    case 8: launch_deep_n<MODE, 8>(a, st, npt); break;
    default: launch_deep_n<MODE, kFoldMaxTiles>(a, st, npt); break;   // drive folded
  }
}

hipError_t launch_fused(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  const int path = sel_path(p), npt = npt_of(p);
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
  if (p.in_bf16 && p.mma_bf16) {
    if (path == kSelBF16D128N3 && npt == 32)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N3, 32, true>(a, st);
    else if (path == kSelBF16D128N3)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N3, 0, true>(a, st);
    else if (path == kSelBF16D128N5 && npt == 32)            // drive folded, N = 32
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N5, 32, true>(a, st);
    else if (path == kSelBF16D128N5)
      launch_kernel<kModeFused, 1, 1, kSelBF16D128N5, 0, true>(a, st);
    else if (path > kSelDeep)
      launch_deep<kModeFused>(a, st, path - kSelDeep, npt);
    else if (npt == 64)
      launch_kernel<kModeFused, 1, 1, kSelAny, 64, true>(a, st);
    else
      launch_kernel<kModeFused, 1, 1, kSelAny, 0, true>(a, st);
  } else if (p.in_bf16) {
    launch_kernel<kModeFused, 1, 0, kSelAny, 0, true>(a, st);
  } else if (path == kSelF32D64N2) {
    if (npt == 16) launch_kernel<kModeFused, 0, 0, kSelF32D64N2, 16, false>(a, st);
    else launch_kernel<kModeFused, 0, 0, kSelF32D64N2, 0, false>(a, st);
  } else if (path == kSelF32D16N1) {
    if (npt == 8) launch_kernel<kModeFused, 0, 0, kSelF32D16N1, 8, false>(a, st);
    else launch_kernel<kModeFused, 0, 0, kSelF32D16N1, 0, false>(a, st);
  } else {
    launch_kernel<kModeFused, 0, 0, kSelAny, 0, true>(a, st);
  }
  return hipGetLastError();
}

}  // namespace pdscan

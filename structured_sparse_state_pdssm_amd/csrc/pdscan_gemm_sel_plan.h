// Which selections run on the all-heads GEMM (pdscan_gemm_sel.h): u shared by
// the heads, in bf16, with one tile of score rows (K <= 32), at most two of
// pre-activation rows (N <= 64, a multiple of 4 for the 16-byte stores of D)
// and whole 64-channel blocks (d a multiple of 64).
#pragma once

namespace pdscan {

inline bool gemm_sel_fits(int u_shared, int in_bf16, int N, int K, int d) {
  return u_shared && in_bf16 && K >= 1 && K <= 32 && N >= 4 && N <= 64 && N % 4 == 0 && d >= 64 &&
         d % 64 == 0;
}

}  // namespace pdscan

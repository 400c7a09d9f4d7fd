// Launcher for the all-heads selection GEMM (pdscan_gemm_sel.h): eight die
// classes of token tiles, each tile's heads in consecutive slots of its class.
#include "pdscan_gemm_sel.h"

namespace pdscan {

hipError_t launch_gemm_sel(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  GemmSelArgs g;
  g.u = (const uint16_t*)a.u; g.W_sel = (const uint16_t*)a.W_sel; g.W_d = (const uint16_t*)a.W_d;
  g.b_d = a.b_d; g.dict = a.dict; g.k_out = a.k_out; g.D_out = a.D_out; g.P_out = a.P_out;
  g.B = p.B; g.H = p.H; g.L = p.L; g.N = p.N; g.K = p.K; g.d = p.d;
  const long long ntok = (long long)p.B * p.L;
  g.tiles = (int)((ntok + kGsTok - 1) / kGsTok);
  const long long grid = 8ll * ((g.tiles + 7) / 8) * p.H;
  if (grid > 0x7fffffffll) return hipErrorInvalidValue;
  if (p.N > 32)
    hipLaunchKernelGGL((pdssm_gemm_sel_kernel<2, 0>), dim3((unsigned)grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((pdssm_gemm_sel_kernel<1, 0>), dim3((unsigned)grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

// The drive term Bu = W_b u (a.W_b [H,N,d]) into Bu [B,H,L,N], on the same
// tiles and die order.
hipError_t launch_gemm_drive(const Args& a, float* Bu, hipStream_t st) {
  const Plan& p = a.p;
  GemmSelArgs g = {};
  g.u = (const uint16_t*)a.u; g.W_d = (const uint16_t*)a.W_b; g.D_out = Bu;
  g.B = p.B; g.H = p.H; g.L = p.L; g.N = p.N; g.K = p.K; g.d = p.d;
  const long long ntok = (long long)p.B * p.L;
  g.tiles = (int)((ntok + kGsTok - 1) / kGsTok);
  const long long grid = 8ll * ((g.tiles + 7) / 8) * p.H;
  if (grid > 0x7fffffffll) return hipErrorInvalidValue;
  if (p.N > 32)
    hipLaunchKernelGGL((pdssm_gemm_sel_kernel<2, 1>), dim3((unsigned)grid), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((pdssm_gemm_sel_kernel<1, 1>), dim3((unsigned)grid), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace pdscan

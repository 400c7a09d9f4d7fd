// Launch plan of the soft-selection comparison pass (the original PD-SSM
// selection: a convex combination of dense dictionary matrices followed by a
// column hardmax) and the arguments one launch reads (host and device).
#pragma once

#include "pdscan_plan.h"

namespace pdscan {

constexpr int kSoftSteps = 1024;   // steps per workgroup (16 per wave and pass)
constexpr int kSoftMaxK = 16;      // dictionary matrices
constexpr int kSoftMaxN = 16;      // state size
constexpr int kSoftMaxD = 128;     // input channels

struct SoftPlan {
  int B, H, L, N, K, d, u_shared, in_bf16;
  int blocks_per_seq, tasks;
  int bytes;
};

inline bool make_soft_plan(SoftPlan& q, int B, int H, int L, int N, int K, int d, int u_shared,
                           int in_bf16) {
  q.B = B; q.H = H; q.L = L; q.N = N; q.K = K; q.d = d; q.u_shared = u_shared; q.in_bf16 = in_bf16;
  q.blocks_per_seq = (L + kSoftSteps - 1) / kSoftSteps;
  q.tasks = q.blocks_per_seq * B * H;
  q.bytes = 0;                                     // registers only, no LDS
  // per-sequence byte ranges addressed with 32-bit offsets
  const bool fits = (size_t)L * N * N * 4 < (size_t)0x80000000u && (size_t)L * d * 4 < (size_t)0x80000000u;
  return N <= kSoftMaxN && K <= kSoftMaxK && (d == 16 || d == 32 || d == 64 || d == 128) && fits;
}

struct SoftArgs {
  SoftPlan q;
  const void* u;        // [B,H,L,d] or [B,L,d]
  const void* W_sel;    // [H,K,d]
  const float* M;       // [H,K,N,N]: M[h,k,i,j], row i, column j
  const void* W_d;      // [H,N,d]
  const float* b_d;     // [H,N]
  float* M_t;           // [B,H,L,N,N] out: the mixtures, materialised
  int32_t* P_idx;       // [B,H,L,N] out: row of column j's one
  float* D;             // [B,H,L,N] out
};

}  // namespace pdscan

// Launch plan of the soft-selection comparison pass (the original PD-SSM
// selection: a convex combination of dense dictionary matrices followed by a
// column hardmax) and the arguments one launch reads (host and device).
#pragma once

#include "pdscan_plan.h"

namespace pdscan {

constexpr int kSoftRows = 16;      // steps per pass of a workgroup (one 16-lane group each)
constexpr int kSoftSteps = 64;     // steps per workgroup
constexpr int kSoftMaxK = 16;      // dictionary matrices
constexpr int kSoftMaxN = 16;      // state size
constexpr int kSoftMaxD = 128;     // input channels

struct SoftPlan {
  int B, H, L, N, K, d, u_shared, in_bf16;
  int blocks_per_seq, tasks;
  int off_u, off_M, off_W, off_a, bytes;
};

inline bool make_soft_plan(SoftPlan& q, int B, int H, int L, int N, int K, int d, int u_shared,
                           int in_bf16) {
  q.B = B; q.H = H; q.L = L; q.N = N; q.K = K; q.d = d; q.u_shared = u_shared; q.in_bf16 = in_bf16;
  q.blocks_per_seq = (L + kSoftSteps - 1) / kSoftSteps;
  q.tasks = q.blocks_per_seq * B * H;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off = align_up(off + bytes, 16); return o; };
  q.off_u = take(kSoftRows * d * 4);               // the block's input rows (fp32)
  q.off_M = take(K * N * N * 4);                   // the head's dense dictionary matrices
  q.off_W = take((K + N) * d * 4);                 // W_sel then W_d rows of the head (fp32)
  q.off_a = take(kSoftRows * kSoftMaxK * 4);       // mixture weights per row
  q.bytes = off;
  return N <= kSoftMaxN && K <= kSoftMaxK && d <= kSoftMaxD && q.bytes <= kMaxLds;
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

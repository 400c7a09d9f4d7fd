// Soft-selection comparison pass (device code): the original PD-SSM
// selection ("Flash PD-SSM" summary, background on the original model:
// every step forms a convex combination of dense N x N dictionary matrices
// and sparsifies it with a column hardmax, which materialises an N x N
// matrix per step, O(L N^2) memory).  Per step t of a (b, h) sequence:
//   alpha_t = softmax(W_sel u_t) over the K matrices,
//   M_t = sum_k alpha_t[k] M[h,k],  written out whole,
//   P_idx_t[j] = the lowest row i with M_t[i, j] = max_i' M_t[i', j],
//   D_t = sigmoid(W_d u_t + b_d).
// The scan then runs on the per-step maps (pdssm_scan_fwd_pidx).
#pragma once

#include "pdscan_device.h"
#include "pdscan_soft_plan.h"

namespace pdscan {

// Stage n values (fp32, or bf16 widened) into LDS: each lane issues a batch
// of buffer loads before storing (base uniform in the workgroup).
__device__ __forceinline__ void soft_stage(float* dst, const void* src, size_t base, int n, int bf16) {
  const int es = bf16 ? 2 : 4;
  const rsrc_t r = make_rsrc((const unsigned char*)src + base * es, (uint32_t)(n * es));
  for (int e0 = 0; e0 < n; e0 += kThreads * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads + (int)threadIdx.x;
      const uint32_t off = e < n ? (uint32_t)(e * es) : kNoLoad;
      v[u] = bf16 ? __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16)
                  : buf_f32(r, off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads + (int)threadIdx.x;
      if (e < n) dst[e] = v[u];
    }
  }
}

// Column hardmax of every dense dictionary matrix: dict[h,k,j] = the lowest
// row i with M[h,k,i,j] maximal (the sparse dictionary of the hard-selection
// path built from dense parameters; same summary, methodology item 1).
__global__ void pdssm_dict_hardmax_kernel(const float* M, int32_t* dict, int HK, int N) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= HK * N) return;
  const int hk = e / N, j = e - hk * N;
  const float* col = M + (size_t)hk * N * N + j;
  int best = 0;
  float bv = col[0];
  for (int i = 1; i < N; ++i)
    if (col[i * N] > bv) {
      bv = col[i * N];
      best = i;
    }
  dict[e] = best;
}

// One workgroup: kSoftSteps consecutive steps of one sequence, 16 at a time;
// lane group r (16 lanes) owns step t0 + r, lane j of it owns column j.
__global__ __launch_bounds__(kThreads) void pdssm_soft_kernel(SoftArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const SoftPlan& q = a.q;
  const int tid = threadIdx.x;
  const int N = q.N, K = q.K, d = q.d, L = q.L;
  const int task = blockIdx.x;
  const int s = task / q.blocks_per_seq;
  const int tblk = (task - s * q.blocks_per_seq) * kSoftSteps;
  const int b = s / q.H, h = s % q.H;
  float* ul = (float*)(smem + q.off_u);            // [16][d]
  float* Ml = (float*)(smem + q.off_M);            // [K][N][N]
  float* Wl = (float*)(smem + q.off_W);            // [K + N][d]
  float* al = (float*)(smem + q.off_a);            // [16][16]

  // ---- the head's parameters, once per workgroup
  soft_stage(Ml, a.M, (size_t)h * K * N * N, K * N * N, 0);
  soft_stage(Wl, a.W_sel, (size_t)h * K * d, K * d, q.in_bf16);
  soft_stage(Wl + K * d, a.W_d, (size_t)h * N * d, N * d, q.in_bf16);
  const int r = tid >> 4, j = tid & 15;
  const float bdj = j < N ? a.b_d[(size_t)h * N + j] : 0.f;

  for (int t0 = tblk; t0 < min(tblk + kSoftSteps, L); t0 += kSoftRows) {
    const int nrow = min(kSoftRows, L - t0);
    __syncthreads();                               // previous rows done with ul and al
    const size_t urow = (size_t)(q.u_shared ? b : s) * L + t0;
    soft_stage(ul, a.u, urow * d, nrow * d, q.in_bf16);
    __syncthreads();

    const bool row_ok = r < nrow;
    const float* ur = ul + r * d;
    // scores (lanes j < K) and pre-activations (lanes j < N), fp32 FMA in
    // channel order
    float sc = 0.f, z = 0.f;
    if (row_ok) {
      const float* ws = Wl + (j < K ? j : 0) * d;
      const float* wz = Wl + (K + (j < N ? j : 0)) * d;
      for (int c = 0; c < d; ++c) {
        sc = __builtin_fmaf(ws[c], ur[c], sc);
        z = __builtin_fmaf(wz[c], ur[c], z);
      }
    }
    // softmax over the K scores of the row (16-lane reductions)
    float m = j < K ? sc : -INFINITY;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    const float ex = j < K ? expf(sc - m) : 0.f;
    float sum = ex;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 16);
    al[r * kSoftMaxK + j] = ex / sum;
    __syncthreads();

    if (row_ok && j < N) {
      const size_t row = (size_t)s * L + t0 + r;
      // column j of M_t (mixture in dictionary order), then its hardmax
      // (strictly greater: the lowest row on ties)
      float col[kSoftMaxN];
#pragma unroll
      for (int i = 0; i < kSoftMaxN; ++i) col[i] = 0.f;
      for (int k = 0; k < K; ++k) {
        const float ak = al[r * kSoftMaxK + k];
        const float* mk = Ml + k * N * N + j;
#pragma unroll
        for (int i = 0; i < kSoftMaxN; ++i)
          if (i < N) col[i] = __builtin_fmaf(ak, mk[i * N], col[i]);
      }
      int best = 0;
      float bv = col[0];
#pragma unroll
      for (int i = 1; i < kSoftMaxN; ++i)
        if (i < N && col[i] > bv) {
          bv = col[i];
          best = i;
        }
      float* mt = a.M_t + row * N * N + j;
#pragma unroll
      for (int i = 0; i < kSoftMaxN; ++i)
        if (i < N) mt[i * N] = col[i];
      a.P_idx[row * N + j] = best;
      a.D[row * N + j] = 1.f / (1.f + expf(-(z + bdj)));
    }
  }
}

}  // namespace pdscan

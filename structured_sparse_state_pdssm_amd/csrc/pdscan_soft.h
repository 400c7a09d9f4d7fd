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

// Four consecutive channels of row `row` of a [rows x d] operand (fp32 or
// bf16 widened), as one 16-byte or 8-byte buffer load; `off` is the element
// offset of the first, kNoLoad for zeros.
__device__ __forceinline__ f4v soft_load4(rsrc_t r, uint32_t off, int bf16) {
  if (bf16) {
    const u2v w = __builtin_bit_cast(
        u2v, __builtin_amdgcn_raw_buffer_load_b64(r, off == kNoLoad ? kNoLoad : off * 2, 0, 0));
    return f4v{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xFFFF0000u)};
  }
  return __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(r, off == kNoLoad ? kNoLoad : off * 4, 0, 0));
}

// One workgroup: kSoftSteps consecutive steps of one sequence; each wave takes
// 16 of them at a time, all in registers.  Every contraction runs on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32, fp32 products and accumulation) with
// the weights as the row operand and the 16 steps as the columns, so lane
// (g, c) of the 64 ends with rows 4g..4g+3 of step c:
//   scores:          [K rows x d] x [d x 16 steps]  (row x holds matrix
//                    (x / 4) + 4 (x % 4), so register r of lane group g is
//                    matrix g + 4 r: the mixture's contraction slot),
//   pre-activations: [N rows x d] x [d x 16 steps],
//   mixture, per row i of M_t:  [N columns j x K] x [K x 16 steps],
// the softmax is a 4-register, 4-lane-group reduction, the column hardmax is a
// running maximum over i in each lane, and a lane writes four consecutive
// columns j of a step with one 16-byte store.  The contraction over channels
// takes slot (g, kb) as channel 16 (kb / 4) + 4 g + kb % 4 on both operands,
// so each lane reads four consecutive channels per load.
template <int NKB>   // NKB = d / 4 channel slots
__global__ __launch_bounds__(kThreads) void pdssm_soft_kernel(SoftArgs a) {
  const SoftPlan& q = a.q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = q.N, K = q.K, d = q.d, L = q.L;
  const int task = blockIdx.x;
  const int s = task / q.blocks_per_seq;
  const int tblk = (task - s * q.blocks_per_seq) * kSoftSteps;
  const int b = s / q.H, h = s % q.H;
  const int c16 = lane & 15, g = lane >> 4;
  const int bf = q.in_bf16;
  const int es = bf ? 2 : 4;
  constexpr int NM = NKB / 4;                      // four-channel loads per operand row

  // ---- row operands, once per workgroup: W_sel rows (permuted as above),
  // W_d rows, dictionary fragments (matrix g + 4 kb, row i, column c16)
  f4v wsel[NM], wd[NM];
  {
    const int ks = (c16 >> 2) + 4 * (c16 & 3);
    const rsrc_t sr = make_rsrc((const unsigned char*)a.W_sel + (size_t)h * K * d * es, (uint32_t)(K * d * es));
    const rsrc_t zr = make_rsrc((const unsigned char*)a.W_d + (size_t)h * N * d * es, (uint32_t)(N * d * es));
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      wsel[m] = soft_load4(sr, ks < K ? (uint32_t)(ks * d + 16 * m + 4 * g) : kNoLoad, bf);
      wd[m] = soft_load4(zr, c16 < N ? (uint32_t)(c16 * d + 16 * m + 4 * g) : kNoLoad, bf);
    }
  }
  float mb[kSoftMaxN][kSoftMaxK / 4];             // dictionary fragments: matrix g + 4 kb, row i, column c16
  {
    const rsrc_t mr = make_rsrc(a.M + (size_t)h * K * N * N, (uint32_t)(K * N * N * 4));
#pragma unroll
    for (int i = 0; i < kSoftMaxN; ++i)
#pragma unroll
      for (int kb = 0; kb < kSoftMaxK / 4; ++kb) {
        const int k = g + 4 * kb;
        mb[i][kb] = buf_f32(mr, (i < N && k < K && c16 < N) ? (uint32_t)(((k * N + i) * N + c16) * 4) : kNoLoad);
      }
  }
  float bd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) bd[r] = 4 * g + r < N ? a.b_d[(size_t)h * N + 4 * g + r] : 0.f;

  // per-sequence descriptors: steps past L fall outside them (reads give
  // zeros, writes are dropped)
  const size_t useq = (size_t)(q.u_shared ? b : s) * L;
  const rsrc_t ur = make_rsrc((const unsigned char*)a.u + useq * d * es, (uint32_t)(L * d * es));
  const rsrc_t mtr = make_rsrc(a.M_t + (size_t)s * L * N * N, (uint32_t)(L * N * N * 4));
  const rsrc_t pr = make_rsrc(a.P_idx + (size_t)s * L * N, (uint32_t)(L * N * 4));
  const rsrc_t dr = make_rsrc(a.D + (size_t)s * L * N, (uint32_t)(L * N * 4));
  const bool vec = (N & 3) == 0;                   // whole four-column groups

  const int tend = min(tblk + kSoftSteps, L);
  int t0 = tblk + 16 * wave;
  f4v ub[NM];                                      // column operand: step t0 + c16
#pragma unroll
  for (int m = 0; m < NM; ++m)
    ub[m] = soft_load4(ur, t0 + c16 < tend ? (uint32_t)((t0 + c16) * d + 16 * m + 4 * g) : kNoLoad, bf);

  for (; t0 < tend; t0 += 16 * kWaves) {
    f4v sc = {0.f, 0.f, 0.f, 0.f}, zc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc = __builtin_amdgcn_mfma_f32_16x16x4f32(wsel[m][e], ub[m][e], sc, 0, 0, 0);
        zc = __builtin_amdgcn_mfma_f32_16x16x4f32(wd[m][e], ub[m][e], zc, 0, 0, 0);
      }
    // the next 16 steps' inputs, in flight during the rest of this pass
    const int tn = t0 + 16 * kWaves;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      ub[m] = soft_load4(ur, tn + c16 < tend ? (uint32_t)((tn + c16) * d + 16 * m + 4 * g) : kNoLoad, bf);

    // softmax over the K matrices of step t0 + c16: register r of lane group
    // g is matrix g + 4 r
    float al[4];
    {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (g + 4 * r < K) mx = fmaxf(mx, sc[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        al[r] = g + 4 * r < K ? expf(sc[r] - mx) : 0.f;
        sum += al[r];
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const float inv = 1.f / sum;
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] *= inv;
    }

    // mixture, row by row: lane (g, c16) gets M_t[t0 + c16][i][4 g + r]; the
    // running column maximum (strictly greater: the lowest row on ties)
    const int t = t0 + c16;
    const uint32_t rowo = (uint32_t)t * N;         // element offset of step t's first row/entry
    f4v best = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int bi[4] = {0, 0, 0, 0};
    uint32_t ob = (rowo * N + 4 * g) * 4;          // byte offset of M_t[t][i][4 g], row i = 0
    const uint32_t ostep = (uint32_t)N * 4;
#pragma unroll
    for (int i = 0; i < kSoftMaxN; ++i) {
      if (i < N) {                                 // a guard, not an exit: every index stays constant
        f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kSoftMaxK / 4; ++kb)
          if (4 * kb < K) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mb[i][kb], al[kb], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (acc[r] > best[r]) {
            best[r] = acc[r];
            bi[r] = i;
          }
        const uint32_t o = ob / 4;                  // M_t element [t][i][4 g]
        if (vec) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v, acc), mtr, 4 * g < N ? ob : kNoLoad, 0, 0);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), mtr,
                                                  4 * g + r < N ? (o + r) * 4 : kNoLoad, 0, 0);
        }
        ob += ostep;
      }
    }
    f4v dv;
#pragma unroll
    for (int r = 0; r < 4; ++r) dv[r] = 1.f / (1.f + expf(-(zc[r] + bd[r])));
    const uint32_t o = rowo + 4 * g;               // P_idx / D element [t][4 g]
    if (vec) {
      const uint32_t ob = 4 * g < N ? o * 4 : kNoLoad;
      __builtin_amdgcn_raw_buffer_store_b128(u4v{(uint32_t)bi[0], (uint32_t)bi[1], (uint32_t)bi[2], (uint32_t)bi[3]},
                                             pr, ob, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v, dv), dr, ob, 0, 0);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ob = 4 * g + r < N ? (o + r) * 4 : kNoLoad;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)bi[r], pr, ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dv[r]), dr, ob, 0, 0);
      }
    }
  }
}

}  // namespace pdscan

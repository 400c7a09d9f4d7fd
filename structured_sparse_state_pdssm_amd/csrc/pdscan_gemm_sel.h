// Selection of a multi-head layer as one GEMM over all tokens: input u
// [B,L,d] shared by the heads, bf16, with the scores and pre-activations of
// the Flash PD-SSM summary's Methodology 1 (s_t = W_sel u_t, argmax with ties
// to the lowest index; D_t = sigmoid(W_d u_t + b_d)) for every head, in the
// layer shape of its Methodology 4.
//
// The per-(chunk, head) selection of the fused kernels reads each token's u
// once per head and each head's weights once per chunk; here a workgroup owns
// 256 tokens of one head, the 24-odd heads of one token tile run on the same
// die (workgroup i runs on die i mod 8), so the tile is fetched from HBM once
// and read by every head from that die's L2.
//
// Tiles.  v_mfma_f32_32x32x16_bf16 with A = 32 weight rows x 16 channels and
// B = 16 channels x 32 tokens: lane l of the output holds token l % 32 and
// weight rows 8 (v / 4) + 4 (l / 32) + v % 4 of accumulator element v.  Row
// tile 0 holds the K <= 32 score rows (rows >= K are zero and skipped by the
// argmax), tiles 1 and 2 the N <= 64 pre-activation rows.  Each wave owns 64
// tokens (two column tiles); the four waves share the weight rows of each
// 64-channel block, staged through LDS in 144-byte rows (two stages); each
// wave's u rows pass through LDS rows of its own, so that the loads read
// whole 128-byte lines while the B operands keep the MFMA lane layout.
//
// Epilogue: the argmax runs over a lane's 16 score rows in increasing row
// order (strict >, so the lowest index wins a tie) and is joined with lane
// l ^ 32, which holds the other 16; the pre-activations get b_d and the
// logistic and leave as 16-byte stores of four consecutive n (the partial
// lines meet in L2; staging them through LDS into whole rows measured no
// faster, and non-temporal stores, which skip that merge, far slower).
#pragma once

#include <hip/hip_runtime.h>

#include "pdscan_device.h"
#include "pdscan_gemm_sel_plan.h"

namespace pdscan {

constexpr int kGsTok = 256;          // tokens per workgroup
constexpr int kGsRowB = 144;         // LDS bytes per staged weight row (64 channels + 16 bytes of padding)

struct GemmSelArgs {
  const uint16_t* u;      // [B*L, d] bf16
  const uint16_t* W_sel;  // [H, K, d] bf16
  const uint16_t* W_d;    // [H, N, d] bf16
  const float* b_d;       // [H, N]
  const int32_t* dict;    // [H, K, N] (P_idx only)
  int32_t* k_out;         // [B, H, L]
  float* D_out;           // [B, H, L, N]
  int32_t* P_out;         // [B, H, L, N] or null
  int B, H, L, N, K, d;
  int tiles;              // token tiles of kGsTok
};

// DRIVE = 0: the selection (score tile, then NDT tiles of pre-activation
// rows; k* and D written).  DRIVE = 1: the drive term Bu = W_b u alone (W_d
// holds W_b [H,N,d], D_out receives Bu [B,H,L,N]; NDT tiles of rows, no
// score tile, no nonlinearity).
template <int NDT, int DRIVE>   // tiles of N rows (N <= 32 NDT)
__global__ __launch_bounds__(256, 2) void pdssm_gemm_sel_kernel(GemmSelArgs a) {
  constexpr int ST = DRIVE ? 0 : 1;              // score tiles
  constexpr int NT = ST + NDT;                   // row tiles
  constexpr int R = 32 * NT;                     // staged weight rows
  __shared__ __attribute__((aligned(16))) unsigned char wl[2][R * kGsRowB];
  __shared__ __attribute__((aligned(16))) unsigned char ul[4][64 * kGsRowB];   // each wave's tokens
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, N = a.N, K = a.K, d = a.d;
  // die-aware order: the heads of token tile T run on die T mod 8
  const int g = blockIdx.x, x = g & 7, q = g >> 3;
  const int T = 8 * (q / H) + x, h = q % H;
  if (T >= a.tiles) return;                      // uniform in the workgroup
  const long long ntok = (long long)a.B * a.L;
  const int nb = d / 64;                         // channel blocks

  // weight rows of this head: a 16-byte piece per thread and pass
  const rsrc_t wsr = make_rsrc(a.W_sel + (DRIVE ? 0 : (size_t)h * K * d), DRIVE ? 0u : (uint32_t)(K * d * 2));
  const rsrc_t wdr = make_rsrc(a.W_d + (size_t)h * N * d, (uint32_t)(N * d * 2));
  u4v ws[NT];
  auto stage_load = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int qq = tid + 256 * m, row = qq >> 3, seg = qq & 7;
      const bool score = m < ST;
      const int wr = score ? row : row - 32 * ST;   // score row, or row n of W_d (W_b)
      const bool ok = score ? wr < K : wr < N;
      const uint32_t off = ok ? (uint32_t)((wr * d + 64 * kb + 8 * seg) * 2) : kNoLoad;
      ws[m] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(score ? wsr : wdr, off, 0, 0));
    }
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int qq = tid + 256 * m, row = qq >> 3, seg = qq & 7;
      *(u4v*)(wl[buf] + row * kGsRowB + seg * 16) = ws[m];
    }
  };

  // this wave's tokens: two column tiles of 32
  const long long t0 = (long long)T * kGsTok + 64 * wave;
  const rsrc_t ur = make_rsrc(a.u + t0 * d, (uint32_t)(ntok - t0 > 0 ? min(ntok - t0, 64ll) * d * 2 : 0));
  const int col = lane & 31, kh = lane >> 5;
  // u of one block: 64 tokens x 128 bytes per wave, loaded with eight lanes
  // per token row (whole 128-byte lines per instruction) into registers,
  // then written to the wave's own LDS rows, from which the B operands are
  // read (lane l: token l % 32 of column tile s, channels 16 ks + 8 (l / 32))
  u4v Ur[8];
  unsigned char* uw = ul[wave];
  auto u_load = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      Ur[i] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                          ur, (uint32_t)(((8 * i + (lane >> 3)) * d + 64 * kb + 8 * (lane & 7)) * 2),
                                          0, 0));
  };
  auto u_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u4v*)(uw + (8 * i + (lane >> 3)) * kGsRowB + (lane & 7) * 16) = Ur[i];
  };

  f16v acc[2][NT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[s][j] = f16v{};
  auto mma_blk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u4v U[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) U[s] = *(const u4v*)(uw + (32 * s + col) * kGsRowB + (16 * ks + 8 * kh) * 2);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u4v w = *(const u4v*)(wl[buf] + (32 * j + col) * kGsRowB + (16 * ks + 8 * kh) * 2);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc[s][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, w),
                                                              __builtin_bit_cast(bf8v, U[s]), acc[s][j], 0, 0, 0);
      }
    }
  };

  // Pipeline, one block deep: while block b multiplies, the weights and u of
  // block b + 1 arrive in registers; they go to LDS after the block's reads
  // (the wave's own u rows need no barrier: one wave's LDS accesses run in
  // order; the shared weight stage alternates and a barrier ends each block).
  stage_load(0);
  u_load(0);
  stage_store(0);
  u_store();
  __syncthreads();
  for (int kb = 0; kb < nb; ++kb) {
    const bool more = kb + 1 < nb;
    if (more) {
      stage_load(kb + 1);
      u_load(kb + 1);
    }
    mma_blk(kb & 1);
    if (more) {
      u_store();
      stage_store((kb + 1) & 1);
    }
    __syncthreads();
  }

  // ---- epilogue
  if constexpr (DRIVE) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const long long t = t0 + 32 * s + col;
      if (t < ntok) {
        const uint32_t b = (uint32_t)t / (uint32_t)a.L, l = (uint32_t)t % (uint32_t)a.L;
        float* dst = a.D_out + (((size_t)b * H + h) * a.L + l) * N;
#pragma unroll
        for (int j = 0; j < NDT; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int n = 32 * j + 8 * v4 + 4 * kh;
            if (n < N)
              *(f4v*)(dst + n) = f4v{acc[s][j][4 * v4], acc[s][j][4 * v4 + 1], acc[s][j][4 * v4 + 2],
                                     acc[s][j][4 * v4 + 3]};
          }
      }
    }
    return;
  }
  float bd[NDT][16];
  {
    const rsrc_t br = make_rsrc(a.b_d + (size_t)h * N, (uint32_t)(N * 4));
#pragma unroll
    for (int j = 0; j < NDT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int n = 32 * j + 8 * (v >> 2) + 4 * kh + (v & 3);
        bd[j][v] = buf_f32(br, n < N ? (uint32_t)n * 4u : kNoLoad);
      }
  }
  const rsrc_t dr = make_rsrc(a.dict + (size_t)h * K * N, a.P_out ? (uint32_t)(K * N * 4) : 0u);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const long long t = t0 + 32 * s + col;       // this lane's token
    const bool live = t < ntok;
    // token counts below 2^31 (checked by the caller): 32-bit division
    const uint32_t b = live ? (uint32_t)t / (uint32_t)a.L : 0u, l = live ? (uint32_t)t % (uint32_t)a.L : 0u;
    const size_t seq = ((size_t)b * H + h) * a.L + l;   // index of (b, h, l)
    // argmax over the lane's 16 score rows, then over the pair of lanes
    float best = 0.f;
    int bi = -1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * kh + (v & 3);
      const float sc = acc[s][0][v];
      if (r < K && (bi < 0 || sc > best)) {
        best = sc;
        bi = r;
      }
    }
    const float ob = __shfl_xor(best, 32, 64);
    const int oi = __shfl_xor(bi, 32, 64);
    if (oi >= 0 && (bi < 0 || ob > best || (ob == best && oi < bi))) {
      best = ob;
      bi = oi;
    }
    if (live && kh == 0) a.k_out[seq] = bi;
    // logistic of the pre-activations; four consecutive n per 16-byte store
#pragma unroll
    for (int j = 0; j < NDT; ++j)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int n = 32 * j + 8 * v4 + 4 * kh;
        if (live && n < N) {
          f4v o;
          o.x = logistic(acc[s][1 + j][4 * v4 + 0] + bd[j][4 * v4 + 0]);
          o.y = logistic(acc[s][1 + j][4 * v4 + 1] + bd[j][4 * v4 + 1]);
          o.z = logistic(acc[s][1 + j][4 * v4 + 2] + bd[j][4 * v4 + 2]);
          o.w = logistic(acc[s][1 + j][4 * v4 + 3] + bd[j][4 * v4 + 3]);
          *(f4v*)(a.D_out + seq * N + n) = o;
          if (a.P_out) {
            i4v pi;
            pi.x = buf_i32(dr, (uint32_t)((bi * N + n + 0) * 4));
            pi.y = buf_i32(dr, (uint32_t)((bi * N + n + 1) * 4));
            pi.z = buf_i32(dr, (uint32_t)((bi * N + n + 2) * 4));
            pi.w = buf_i32(dr, (uint32_t)((bi * N + n + 3) * 4));
            *(i4v*)(a.P_out + seq * N + n) = pi;
          }
        }
      }
  }
}

}  // namespace pdscan

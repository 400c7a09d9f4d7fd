// Launch plan of the impulse-sensitivity pass (dy_t / du_0 for fixed
// selections): tiling, on-chip layout, workspace layout and the arguments one
// launch reads (host and device).
#pragma once

#include "pdscan_plan.h"

namespace pdscan {


constexpr int kSensMaxD = 128;   // input channels (multiple of 16)
constexpr int kSensWin = 8;      // later-published chunks one window read covers
constexpr int kSensRow = 16;     // LDS row width of the weight rows (N <= 16)
constexpr int kSensMaxS = 32;    // steps per lane group at most (chunk <= 512)

struct SensPlan {
  int B, H, L, N, K, d, in_bf16, chunk;
  int S, G, GS, nC, tasks;
  int spin_limit, force_giveup;   // look-back give-up, as in Plan
  int off_dk, off_C, off_k, off_W, off_cb, off_P, off_V, off_win, off_misc, bytes;
  size_t ws_agg, ws_inc, ws_bytes;
};

inline bool make_sens_plan(SensPlan& q, int B, int H, int L, int N, int K, int d, int in_bf16,
                           int chunk) {
  q.B = B; q.H = H; q.L = L; q.N = N; q.K = K; q.d = d; q.in_bf16 = in_bf16;
  q.chunk = chunk < L ? chunk : L;
  q.spin_limit = kSpinLimit;
  q.force_giveup = 0;
  q.G = kThreads / 16;
  q.S = align_up((q.chunk + q.G - 1) / q.G, 4);
  q.GS = q.S * kSensRow + kSensRow;               // group stride, 16 (mod 64) words
  q.nC = (L + q.chunk - 1) / q.chunk;
  q.tasks = q.nC * B * H;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off = align_up(off + bytes, 16); return o; };
  q.off_dk = take(K * 8);
  q.off_C = take(kSensRow * 4);
  q.off_k = take(q.S * q.G * 4);
  q.off_W = take((q.G * q.GS + 8 * kSensRow) * 4);   // + 8 rows of slack for block reads
  q.off_cb = take(kSensRow * 4);                     // step-0 coefficients
  q.off_P = take(4 * q.G * kSensRow * 4);            // combine: sP, sS, pP, pS
  q.off_V = take(4 * q.G * kSensRow * 4);            // per-group maps of phase C
  q.off_win = take((kSensWin * (4 * kSensRow + 1) + 4 * kSensRow) * 4);   // window, E and F maps
  q.off_misc = take(16);
  q.bytes = off;
  const size_t seqchunks = (size_t)q.nC * B * H;
  q.ws_agg = 256;
  q.ws_inc = q.ws_agg + seqchunks * 2 * N * sizeof(uint64_t);
  q.ws_bytes = q.ws_inc + seqchunks * 2 * N * sizeof(uint64_t);
  return q.S <= kSensMaxS && q.bytes <= kMaxLds;
}

struct SensArgs {
  SensPlan q;
  const int32_t* k_star;
  const int32_t* dict;
  const float* D;
  const void* W_d;   // [H,N,d], fp32 or bf16
  const void* W_b;   // [H,N,d], fp32 or bf16
  const float* C;
  const float* h0;   // [B,H,N] or null
  float* dY;         // [B,H,L,d]
  unsigned char* ws;
};

}  // namespace pdscan

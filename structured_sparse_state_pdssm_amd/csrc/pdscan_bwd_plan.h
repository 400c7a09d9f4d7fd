// Launch plan of the gradient pass through the scan: on-chip layout and the
// arguments one launch reads (host and device).
#pragma once

#include "pdscan_plan.h"

namespace pdscan {

// Later chunks whose carries and maps the look-back reads in one batch.
constexpr int kBwdLookWin = 8;

// LDS byte offsets of the backward kernel.
struct BwdLds {
  int off_dic, off_dk, off_D, off_k, off_gy, off_C, off_s, off_p, off_slot, off_H, off_gc, off_win, off_misc, bytes;
  // word stride between the lane groups' D rows: S*N, plus NP when that is a
  // multiple of 64, so the groups of one half-wave reading their step i do
  // not all land on the same banks
  int GS;
};

// `p` is the forward scan plan with the same chunk: groups, steps per group,
// and the workspace words of the chunk carries.  Returns false when the
// layout needs more than kMaxLds bytes.
inline bool make_bwd_lds(const Plan& p, BwdLds& l) {
  const int N = p.N, K = p.K, T = p.chunk, G = p.G;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off = align_up(off + bytes, 16); return o; };
  l.off_dic = take(K * N * 4);
  l.off_dk = take(K * 8);        // N <= 16: each dictionary row as 16 nibbles
  l.GS = p.S * N;
  if (p.NP < 64 && l.GS % 64 == 0) l.GS += p.NP;
  l.off_D = take((G * l.GS + 16 * N) * 4);   // 8 rows of slack on each side (block reads past a group's ends)
  l.off_k = take(T * 4);
  l.off_gy = take(T * 4);
  l.off_C = take(N * 4);
  l.off_s = take(3 * G * N * 4);
  l.off_p = take(3 * G * N * 4);
  l.off_slot = take(kThreads * 4);
  l.off_H = take(64 * 4);
  l.off_gc = take(G * N * 4);
  l.off_win = take(kBwdLookWin * (4 * N + 1) * 4);   // look-back window: maps, carries, flags
  l.off_misc = take(16);
  l.bytes = off;
  return l.bytes <= kMaxLds;
}

struct BwdArgs {
  Plan p;        // geometry of the forward scan with the same chunk
  BwdLds l;
  size_t ws_gc;  // workspace byte offset of the per-task dC partials [nC][B*H][N]
  const int32_t* k_star;
  const int32_t* dict;
  const float* D;
  const float* C;
  const float* h0;
  const float* H_all;
  const float* g_y;
  const float* g_hL;
  float* g_Bu;
  float* g_D;
  float* g_h0;
  unsigned char* ws;
};

// Workspace of the gradient pass: the forward scan's (header, maps and
// carries, reused with the adjoint meaning) and the dC partials after it.
inline size_t bwd_ws_gc(const Plan& p) { return (p.ws_bytes + 255) / 256 * 256; }
inline size_t bwd_ws_bytes(const Plan& p) {
  return bwd_ws_gc(p) + (size_t)p.nC * p.B * p.H * p.N * sizeof(float);
}

}  // namespace pdscan

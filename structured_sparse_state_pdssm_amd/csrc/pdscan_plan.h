// Launch plan shared by the host dispatcher and the kernels: work split,
// on-chip (LDS) layout and workspace layout for one call.
//
// Work split.  One workgroup (256 lanes, 4 waves) owns one chunk of one
// (b, h) sequence.  Inside it the chunk's steps are cut into G consecutive
// sub-chunks of S steps, one per lane group; a lane group is NP = next power
// of two >= N lanes, so each lane owns one state row and G * NP = 256.
// Phase A runs the G sub-chunks side by side; their summaries are combined in
// order in LDS to form the chunk summary that enters the inter-chunk scan.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pdscan {

constexpr int kThreads = 256;          // lanes per workgroup
constexpr int kWaves = kThreads / 64;  // wave64
constexpr int kSelectRows = 256;       // rows per workgroup for selection alone
constexpr int kMaxLds = 64 * 1024;     // bytes of LDS one workgroup uses on the established paths (2 per CU)
constexpr int kMaxLdsGfx950 = 160 * 1024;   // the whole LDS of one gfx950 CU: one workgroup may take all of it
constexpr int kFoldMaxTiles = 10;      // general kernel, drive folded: column tiles of the selection GEMM
constexpr int kWbFrags = 6;            // W_b fragments per lane at most (fp32 d = 64: 2 blocks x 3 pieces)
constexpr int kMaxOut = 4;             // outputs per head (rows of C) on the multi-output paths
constexpr int kSpinLimit = 1 << 22;    // window reads before a look-back wait gives up
constexpr int kXcds = 8;               // accelerator dies (XCDs); workgroup i is dispatched to die i mod 8
constexpr double kL2WeightBudget = 2.5 * 1024 * 1024;   // bytes of one die's 4 MiB L2 the weights may hold

enum Mode : int { kModeSelect = 0, kModeScan = 1, kModeFused = 2 };

struct Plan {
  // problem
  int B, H, L, N, K, d, u_shared, in_bf16, chunk;
  // work split
  int NP;    // lanes per group
  int G;     // groups per workgroup
  int S;     // steps per group (a multiple of 4)
  int TS;    // row stride of the on-chip [N][TS] diagonal / output-weight buffer
  int skew;  // 1: step t of group g sits in column t + g (fused16 layout)
  int DCS;   // row stride of the (row, C[row]) dictionary table
  int nC;    // chunks per sequence
  int NC;    // GEMM columns (K scores then N pre-activations), padded to 16
  int KP;    // score staging width
  int mma_bf16;  // score GEMM on bf16 MFMA (else fp32 MFMA)
  int fused16;   // fused pass with step-major MFMA tiles (N, K <= 16; see below)
  int fold_bu;   // Bu = W_b u formed on chip instead of read: a third MFMA tile (fused16) or a third
                 // column segment of the selection GEMM written to an on-chip [N][TS] buffer (general kernel)
  int step16;    // scan alone with the step-major layout (N <= 16); 2: also writes every state
  int step32;    // general fused kernel with step-major selection tiles (32-lane groups, see below)
  int n_out;     // outputs per head, rows of C (> 1: step-major paths only)
  int gse;       // general kernel, N = 32 or 64: phase A gathers over inverse dictionary rows (table at off_SRC)
  int wst;       // fused deep bf16 selection: weight blocks staged through LDS (in D's region);
                 // 2: in 64-channel blocks
  int YS;        // stride of the per-output local-output rows
  int tasks;     // workgroups
  int xhg;       // general fused kernel: head groups of the die grouping (0: one ticket counter; see
                 // xcd_head_groups)
  // look-back: window reads before a wait gives up (sets the workspace error
  // word and carries h0), and a test hook that ignores every carry found, so
  // that each wait runs out after spin_limit reads while the kernel still
  // ends normally
  int spin_limit, force_giveup;
  int pmask;     // 0x01010101: the gather's source-presence mask, passed at run time (see gather4w)
  // LDS byte offsets
  int off_D, off_k, off_yl, off_dict, off_DC, off_SRC, off_C, off_bd, off_slot, off_sIdx, off_sSc, off_sB,
      off_pIdx, off_pSc, off_pB, off_H, off_tmp, off_WB, off_Bu, off_misc, lds_bytes;
  int lds_limit;   // the plan's LDS budget (kMaxLds, or kMaxLdsGfx950 for the folded / multi-output general plans)
  // workspace byte offsets (scan / fused)
  size_t ws_agg, ws_inc, ws_bytes;
};

inline int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

inline int align_up(int x, int a) { return (x + a - 1) / a * a; }

inline bool make_plan_once(Plan& p, int mode, int B, int H, int L, int N, int K, int d, int u_shared,
                           int in_bf16, int chunk, int fold_bu, int step16, int n_out, int allow_gse) {
  p.B = B; p.H = H; p.L = L; p.N = N; p.K = K; p.d = d;
  p.u_shared = u_shared; p.in_bf16 = in_bf16;
  p.spin_limit = kSpinLimit;
  p.force_giveup = 0;
  p.pmask = 0x01010101;
  // a chunk longer than the sequence behaves exactly like chunk = L
  p.chunk = (mode == kModeSelect) ? kSelectRows : (chunk < L ? chunk : L);
  // Step-major fused path: 16-lane groups, each MFMA tile holding four steps
  // of each of a wave's four groups, so D and k* land in the lanes that use
  // them.  Per-head inputs, N and K up to 16, the register-resident weight
  // shapes, at most 32 steps per group.
  const int kch = in_bf16 ? (d >= 128 ? (d == 128 ? 4 : 0) : 0) : (d == 16 || d == 32 || d == 64 ? d / 16 : 0);
  p.fused16 = (mode == kModeFused && !u_shared && N <= 16 && K <= 16 && kch > 0 &&
               (chunk < L ? chunk : L) <= 512) ? 1 : 0;
  // the general kernel folds the drive as a third column segment of its
  // selection GEMM (at most kFoldMaxTiles column tiles)
  const int KT = (K + 15) >> 4, NT = (N + 15) >> 4;
  const bool deep_sel = in_bf16 && d % 32 == 0 && d >= 256;   // the deep bf16 selection
  const bool gen_fold = mode == kModeFused && !p.fused16 && fold_bu &&
                        (deep_sel ? ((KT + 2 * NT + 1) & ~1) <= kFoldMaxTiles : align_up(K + 2 * N, 16) <= 128);
  p.fold_bu = ((p.fused16 || gen_fold) && fold_bu) ? 1 : 0;
  // General fused kernel, N = 32: the selection as 32x32 MFMA tiles whose
  // rows are (group, step) pairs, so that D and the scores of a group's steps
  // land in its lanes' registers (per-head bf16 u, d = 128, K <= 16, unfolded,
  // one output, at most two tiles of 16 steps per group: chunk <= 256; the
  // inverse-row gather is required)
  p.step32 = (mode == kModeFused && !p.fused16 && !u_shared && in_bf16 && d == 128 && N == 32 && K <= 16 &&
              !p.fold_bu && n_out == 1 && allow_gse && (chunk < L ? chunk : L) <= 256) ? 1 : 0;
  // the scan alone on the same layout: maps streamed per step (at most 32
  // steps per group, as above)
  p.step16 = (mode == kModeScan && step16 && N <= 16 && K <= 16 && (chunk < L ? chunk : L) <= 512) ? step16 : 0;
  const bool sm = p.fused16 || p.step16;
  p.NP = sm ? 16 : next_pow2(N);
  p.G = kThreads / p.NP;
  p.S = align_up((p.chunk + p.G - 1) / p.G, p.step32 ? 16 : 4);   // step32: whole tiles of 16 steps
  // t-contiguous rows; a stride of 4 (mod 32) words spreads the rows of one
  // column over distinct LDS banks while keeping 16-byte alignment
  // Column layout.  fused16: group g's step t goes to column t + g and the
  // row stride is 2 (mod 32), so the 64 lanes of a wave writing one step of
  // four groups hit 64 distinct banks in every 32-lane half.  Otherwise
  // t-contiguous rows with a stride of 4 (mod 32) for 16-byte accesses.
  p.skew = sm ? 1 : 0;
  if (p.skew) {
    p.TS = p.chunk + p.G;
    p.TS += ((2 - p.TS % 32) + 32) % 32;
  } else {
    p.TS = align_up(p.chunk, 4);
    if (p.TS % 32 != 4) p.TS += (36 - p.TS % 32) % 32;
  }
  p.DCS = sm ? 16 : N + 1;   // the step-major kernels index with a shift
  // general kernel with 32- or 64-row groups: phase A's scatter is a gather
  // over the sources of each row (a per-task table of 8 bytes per dictionary
  // entry and row)
  p.gse = (allow_gse && mode != kModeSelect && !sm && (N == 32 || N == 64)) ? 1 : 0;
  if (p.gse) p.DCS = N;      // the gather path indexes the map rows with a shift
  p.nC = (L + p.chunk - 1) / p.chunk;
  p.NC = align_up(K + N + (p.fold_bu && !sm ? N : 0), 16);   // scores, pre-activations, drive terms
  p.KP = align_up(K, 4);
  p.mma_bf16 = (in_bf16 && d >= 128) ? 1 : 0;
  p.tasks = p.nC * B * H;
  p.xhg = 0;

  const int T = p.chunk;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off = align_up(off + bytes, 16); return o; };
  const bool scan = mode != kModeSelect;
  // multi-output: w_t and the local outputs once per row of C
  p.n_out = n_out;
  p.YS = align_up(T + p.G, 4);
  p.off_D = scan ? take(n_out * N * p.TS * 4) : 0;
  // fused deep bf16 selection (d a multiple of 32, at least 256) in one pass
  // over at most six column tiles with at most 32 rows per wave: two stages
  // of 16 columns x 80 bytes per tile in D's region, if it is large enough
  // (folded: up to kFoldMaxTiles tiles, the drive tiles after the others)
  {
    const int dt = KT + NT + (p.fold_bu && !sm ? NT : 0), nct = (dt + 1) & ~1;
    const bool deep = mode == kModeFused && !sm && in_bf16 && p.mma_bf16 && d % 32 == 0 && d >= 256;
    p.wst = (deep && nct <= (p.fold_bu ? kFoldMaxTiles : 6) && (64 / p.NP) * p.S <= 32 &&
             n_out * N * p.TS * 4 >= 2 * 16 * nct * 80) ? 1 : 0;
    // unfolded, d a multiple of 64: 64-channel blocks (whole 128-byte lines
    // per block) when their stages (144-byte rows) fit as well
    if (p.wst && !p.fold_bu && d % 64 == 0 && n_out * N * p.TS * 4 >= 2 * 16 * nct * 144) p.wst = 2;
  }
  // general kernel, drive folded: the drive terms of the chunk, [N][TS]
  p.off_Bu = (p.fold_bu && !sm) ? take(N * p.TS * 4) : 0;
  p.off_k = (scan && !sm) ? take(align_up(T, 4) * 4) : 0;   // the step-major kernels keep k* in registers
  p.off_yl = scan ? take(n_out * p.YS * 4) : 0;
  p.off_dict = scan ? 0 : take(K * N * 4);   // selection: P_idx gathers
  // step-major: row o of C at 16 o; general kernel: at N o
  p.off_C = take((sm ? (N > 16 * n_out ? N : 16 * n_out) : N * n_out) * 4);
  p.off_bd = take(N * 4);
  p.off_slot = take(kThreads * 4);
  const int gn = p.G * N * 4;                      // one [G][N] scratch array of the steps after phase A
  if (sm) {
    // The dictionary tables and the W_b fragments are read in phase A only
    // (and, when every state is written, again after the carries are known);
    // the combine and look-back scratch is written only after phase A (a
    // barrier separates the two), so without the states replay both share
    // one region.
    const int tabs = K * 16 * 8 + K * 16 * 32 + (p.fold_bu ? kWbFrags * 64 * 16 : 0);
    const int u0 = take(p.step16 == 2 ? tabs + 6 * gn : (tabs > 6 * gn ? tabs : 6 * gn));
    const int s0 = p.step16 == 2 ? u0 + tabs : u0;
    p.off_DC = u0;                                 // (row, C[row]) pairs
    p.off_SRC = u0 + K * 16 * 8;                   // source columns of each row and their weights
    p.off_WB = p.fold_bu ? p.off_SRC + K * 16 * 32 : 0;   // W_b MFMA fragments, one 16-byte slot per lane
    p.off_sIdx = s0;
    p.off_sSc = s0 + gn;
    p.off_sB = s0 + 2 * gn;
    p.off_pIdx = s0 + 3 * gn;
    p.off_pSc = s0 + 4 * gn;
    p.off_pB = s0 + 5 * gn;
  } else {
    p.off_DC = scan ? take(K * p.DCS) : 0;        // scan: target row of each source (a byte)
    p.off_SRC = p.gse ? take(K * N * 8) : 0;      // first eight sources of each row
    p.off_WB = 0;
    p.off_sIdx = scan ? take(gn) : 0;
    p.off_sSc = scan ? take(gn) : 0;
    p.off_sB = scan ? take(gn) : 0;
    p.off_pIdx = scan ? take(gn) : 0;
    p.off_pSc = scan ? take(gn) : 0;
    p.off_pB = scan ? take(gn) : 0;
  }
  p.off_H = take(64 * 4);
  p.off_tmp = take(64 * 4);
  p.off_misc = take(16);
  p.lds_bytes = off;

  // workspace: header (ticket counter, error word) then tagged chunk
  // aggregates (3N words per chunk and sequence) and inclusive states (N).
  const size_t seqchunks = (size_t)p.nC * B * H;
  p.ws_agg = 256;
  p.ws_inc = p.ws_agg + seqchunks * 3 * N * sizeof(uint64_t);
  p.ws_bytes = (mode == kModeSelect) ? 0 : p.ws_inc + seqchunks * N * sizeof(uint64_t);
  // several outputs per head: the step-major paths, and the general kernel in
  // the fused and scan modes
  if (n_out < 1 || n_out > kMaxOut || (n_out > 1 && mode == kModeSelect)) return false;
  // The folded and multi-output general plans may take the whole LDS of a
  // CU (one workgroup per CU); every other plan keeps to kMaxLds, so that
  // two workgroups share a CU.
  p.lds_limit = (!sm && (p.fold_bu || n_out > 1)) ? kMaxLdsGfx950 : kMaxLds;
  return p.lds_bytes <= p.lds_limit;
}

// Die grouping of the general fused kernel.  Each of the eight dies has its
// own L2, and workgroup i runs on die i mod 8, so a workgroup takes its task
// from a ticket counter of its die's class: class x owns the (b, h) sequences
// with b in batch group x / hg and h in head group x mod hg (hg head groups,
// 8 / hg batch groups, contiguous near-equal ranges), in chunk-major order.
// The weights of a head are then read by 8 / hg dies instead of all eight and
// a shared input row u[b, t] by hg dies: hg is picked to minimise the bytes
// the dies fetch beyond their L2, with a head group's weights expected to stay
// in L2 across chunks only when they take at most kL2WeightBudget.  A
// predecessor chunk of a task has a lower ticket of the same counter, so the
// look-back only waits on workgroups that have started.  0 (one counter, the
// plain chunk-major order) when no sharing is worth it or a class would be
// empty.
inline int xcd_head_groups(int B, int H, int L, int N, int K, int d, int u_shared, int in_bf16, int fold,
                           int nC) {
  const double es = in_bf16 ? 2 : 4;
  const double Wt = (double)H * (K + N * (fold ? 2 : 1)) * d * es;   // selection weights of every head
  const double Ut = u_shared ? (double)B * L * d * es : 0.0;          // the shared input
  if (!u_shared && Wt <= 1024.0 * 1024.0) return 0;
  int best = 0;
  double best_cost = 0;
  for (int hg = 1; hg <= kXcds; hg *= 2) {
    const int bg = kXcds / hg;
    if (hg > H || bg > B) continue;
    double cost = hg * Ut + bg * Wt;
    if (Wt / hg > kL2WeightBudget) cost += (nC - 1) * bg * Wt;
    if (!best || cost < best_cost) { best = hg; best_cost = cost; }
  }
  return best;
}

// Workgroups of a plan with hg head groups (0: none): eight classes padded to
// the largest; a workgroup whose ticket is past its class's tasks exits.
inline long long xcd_tasks(const Plan& p, int hg) {
  if (!hg) return (long long)p.nC * p.B * p.H;
  const int bg = kXcds / hg;
  return (long long)kXcds * ((p.B + bg - 1) / bg) * ((p.H + hg - 1) / hg) * p.nC;
}

// Fills `p` for one call.  `mode` selects which parts exist.  Returns false
// when the plan needs more LDS than its budget (lds_limit; the gather table
// is dropped first: phase A then scatters with LDS atomics).
inline bool make_plan(Plan& p, int mode, int B, int H, int L, int N, int K, int d, int u_shared,
                      int in_bf16, int chunk, int fold_bu = 0, int step16 = 0, int n_out = 1) {
  if (make_plan_once(p, mode, B, H, L, N, K, d, u_shared, in_bf16, chunk, fold_bu, step16, n_out, 1))
    return true;
  return p.gse && make_plan_once(p, mode, B, H, L, N, K, d, u_shared, in_bf16, chunk, fold_bu, step16, n_out, 0);
}

// Everything a kernel launch reads.
struct Args {
  Plan p;
  const void* u;
  const void* W_sel;
  const void* W_d;
  const float* b_d;
  const int32_t* dict;
  const float* Bu;
  const void* W_b;       // fold_bu: [H,N,d] in u's dtype
  const float* C;
  const float* h0;
  const int32_t* k_in;   // scan mode
  const int32_t* P_in;   // scan mode, per-step column maps [B,H,L,N] instead of k_in and dict
                         // (the plan's K is then the chunk length: one table entry per step)
  const float* D_in;     // scan mode
  int32_t* k_out;        // optional
  float* D_out;          // optional
  int32_t* P_out;        // optional (selection mode)
  float* y;
  float* hL;
  float* H_all;          // optional (scan mode): the state after every step
  unsigned char* ws;     // workspace base
};

// Workspace header words.
constexpr int kWsTicket = 0;   // uint32 ticket counter
constexpr int kWsError = 1;    // uint32: nonzero if a look-back wait of this call gave up
constexpr int kWsClassTicket = 8;   // uint32 x 8: the die classes' ticket counters (die grouping)

}  // namespace pdscan

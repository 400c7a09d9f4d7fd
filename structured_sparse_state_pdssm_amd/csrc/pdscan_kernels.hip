// HIP kernels for gfx950 (CDNA4): selection, chunked scan, and the fused pass.
//
// One kernel template serves three modes (pdscan_plan.h):
//   select : score GEMM + argmax + logistic, results to global memory
//   scan   : selections read from global memory, then phases A, B, C
//   fused  : score GEMM feeding phases A, B, C on chip (the hot path)
//
// Sources: "Flash PD-SSM: Memory-Optimized Structured Sparse State-Space
// Models" (gist.science explainer), technical summary, methodology item 1
// (hard selection by argmax over K linear scores; the selected matrix is a
// one-hot column selector) and item 3 (phase A: sequential recurrences inside
// chunks; phase B: prefix scan of chunk summaries into carry states; phase C:
// carry correction).  A map (idx, scale) stands for the matrix with
// scale[j] in row idx[j] of column j; applying it is a scatter-add, and two
// maps compose by an index gather and a scale product.
//
// On-chip layout of one chunk (T steps): D and then w live in one [N][TS]
// buffer (t contiguous), so the selection epilogue stores four steps of one
// column with one 16-byte write, phase A reads four steps per lane at once,
// and phase C reads consecutive steps on consecutive lanes.
//
// Phase B is a single-pass decoupled look-back: workgroups take chunk tickets
// in (chunk, sequence) order, publish their chunk aggregate, then walk back
// over predecessors until an inclusive state is found.  Every word published
// to other workgroups is a 64-bit (tag, payload) pair written and read with
// device-scope atomics, so no fences are needed and a reader never sees half
// a record.  Inclusive states are always produced by applying aggregates to a
// state vector in chunk order with the same arithmetic, so the result does
// not depend on how far a look-back had to walk.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pdscan_plan.h"

namespace pdscan {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef int i4v __attribute__((ext_vector_type(4)));
typedef int i2v __attribute__((ext_vector_type(2)));

constexpr uint64_t kTagValid = 1ull << 32;
constexpr int kSpinLimit = 1 << 22;
constexpr int kBuBlock = 32;   // phase-A steps whose drive terms sit in registers

// Compiler-level ordering point between LDS accesses of different lanes of
// one wave.  The hardware executes one wave's LDS instructions in order.
#define WAVE_SYNC()                          \
  do {                                       \
    __atomic_signal_fence(__ATOMIC_SEQ_CST); \
    __builtin_amdgcn_wave_barrier();         \
    __atomic_signal_fence(__ATOMIC_SEQ_CST); \
  } while (0)

__device__ __forceinline__ float logistic(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t payload) {
  __hip_atomic_store(p, kTagValid | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_tagged(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool tag_ok(uint64_t w) { return (w >> 32) == 1u; }

// DPP lane permutations inside 16-lane rows.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// (value, index) pair order: larger value first, then the lower index.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& k) {
  const float ov = dpp_f<CTRL>(v);
  const int ok = dpp_i<CTRL>(k);
  const bool take = (ov > v) || (ov == v && ok < k);
  v = take ? ov : v;
  k = take ? ok : k;
}

// Sum over a lane group of NP lanes (NP a power of two); every lane of the
// group gets the same value.
__device__ __forceinline__ float group_sum(float v, int NP) {
  if (NP >= 2) v += dpp_f<kDppXor1>(v);
  if (NP >= 4) v += dpp_f<kDppXor2>(v);
  if (NP >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (NP >= 16) v += dpp_f<kDppMirror>(v);
  if (NP >= 32) v += __shfl_xor(v, 16, 64);
  if (NP >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Selection of one wave's rows.
//
// MFMA tiles of 16 rows: lane (i = lane%16, g = lane/16) feeds A = u[row0+i][c]
// and B = W[col][c]; fp32 (v_mfma_f32_16x16x4_f32) takes channel m + 4g + q at
// step q of channel block m, bf16 (v_mfma_f32_16x16x32_bf16) channels
// m + 8g .. +7.  Both operands use the same channel order, so each output is
// the full contraction.  acc[ct] holds rows row0 + 4g + r, column 16 ct + i
// of [scores | pre-activations].
//
// FAST = true: W lives in registers for the whole wave (KCH channel blocks,
// NCT column tiles known at compile time) and the next tile's u is loaded
// while the current one is multiplied.  FAST = false: any shape, operands
// loaded per tile.
// ---------------------------------------------------------------------------
struct SelDst {
  int* kbuf;      // chunk-local k* (fused) or nullptr
  float* Dbuf;    // [N][TS] (fused) or nullptr
  int TS;
  int32_t* k_out; // global, optional
  float* D_out;   // global, optional
  int32_t* P_out; // global, optional
  const int* dic; // LDS dictionary [K][N] (for P_out)
  size_t gbase;   // global row index of chunk row 0 = s*L + c0
};

template <int IN_BF16, int MMA_BF16>
struct Frag;
template <>
struct Frag<0, 0> { typedef f4v T; };
template <>
struct Frag<1, 0> { typedef u2v T; };
template <>
struct Frag<1, 1> { typedef u4v T; };

template <int IN_BF16, int MMA_BF16>
__device__ __forceinline__ typename Frag<IN_BF16, MMA_BF16>::T load_frag(const void* base, size_t off,
                                                                         bool ok) {
  typedef typename Frag<IN_BF16, MMA_BF16>::T T;
  T z = {};
  if (!ok) return z;
  if constexpr (!IN_BF16) return *(const T*)((const float*)base + off);
  else return *(const T*)((const uint16_t*)base + off);
}

template <int IN_BF16, int MMA_BF16>
__device__ __forceinline__ void mma_step(f4v& acc, typename Frag<IN_BF16, MMA_BF16>::T a,
                                         typename Frag<IN_BF16, MMA_BF16>::T b) {
  if constexpr (MMA_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a),
                                                  __builtin_bit_cast(bf8v, b), acc, 0, 0, 0);
  } else if constexpr (IN_BF16) {
    const float a0 = __uint_as_float(a.x << 16), a1 = __uint_as_float(a.x & 0xffff0000u);
    const float a2 = __uint_as_float(a.y << 16), a3 = __uint_as_float(a.y & 0xffff0000u);
    const float b0 = __uint_as_float(b.x << 16), b1 = __uint_as_float(b.x & 0xffff0000u);
    const float b2 = __uint_as_float(b.y << 16), b3 = __uint_as_float(b.y & 0xffff0000u);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, b2, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, b3, acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
  }
}

// channels per fragment block: 16 (fp32 MFMA, 4 per lane group) or 32 (bf16)
template <int MMA_BF16>
constexpr int kChanBlock = MMA_BF16 ? 32 : 16;

// Epilogue of one tile: argmax over score columns, logistic of the
// pre-activations, stores.  rows >= rlim are not stored.
template <int NCT>
__device__ __forceinline__ void tile_epilogue(const Plan& p, const f4v* acc, const float* bdr,
                                              int row0, int rlim, int lane, const SelDst& o) {
  const int i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  float bv[4];
  int bk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { bv[r] = -__builtin_inff(); bk[r] = 0x7fffffff; }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ct + i;
    if (col < K) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (acc[ct][r] > bv[r]) { bv[r] = acc[ct][r]; bk[r] = col; }   // columns rise with ct
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    argmax_step<kDppXor1>(bv[r], bk[r]);
    argmax_step<kDppXor2>(bv[r], bk[r]);
    argmax_step<kDppHalfMirror>(bv[r], bk[r]);
    argmax_step<kDppMirror>(bv[r], bk[r]);
  }
  const int rb = row0 + 4 * g;   // first of this lane's four rows
  const bool full = rb + 4 <= rlim;
  if (i == 0) {
    if (o.kbuf) {
      if (full) *(i4v*)(o.kbuf + rb) = i4v{bk[0], bk[1], bk[2], bk[3]};
      else
        for (int r = 0; r < 4; ++r) if (rb + r < rlim) o.kbuf[rb + r] = bk[r];
    }
    if (o.k_out)
      for (int r = 0; r < 4; ++r) if (rb + r < rlim) o.k_out[o.gbase + rb + r] = bk[r];
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ct + i;
    if (col >= K && col < K + N) {
      const int n = col - K;
      f4v dv;
#pragma unroll
      for (int r = 0; r < 4; ++r) dv[r] = logistic(acc[ct][r] + bdr[ct]);
      if (o.Dbuf) {
        float* dst = o.Dbuf + n * o.TS + rb;
        if (full) *(f4v*)dst = dv;
        else
          for (int r = 0; r < 4; ++r) if (rb + r < rlim) dst[r] = dv[r];
      }
      if (o.D_out)
        for (int r = 0; r < 4; ++r)
          if (rb + r < rlim) o.D_out[(o.gbase + rb + r) * N + n] = dv[r];
    }
  }
  if (o.P_out) {
    for (int r = 0; r < 4; ++r)
      for (int gg = 0; gg < 4; ++gg) {
        const int kr = __shfl(bk[r], 16 * gg, 64);
        const int row = row0 + 4 * gg + r;
        if (row < rlim)
          for (int n = lane; n < N; n += 64) o.P_out[(o.gbase + row) * N + n] = o.dic[kr * N + n];
      }
  }
}

template <int IN_BF16, int MMA_BF16, int KCH, int NCT>
__device__ __forceinline__ void select_rows(const Args& a, int s_u, int h, int c0, int rbeg,
                                            int rend, int lane, const SelDst& o) {
  typedef typename Frag<IN_BF16, MMA_BF16>::T FT;
  constexpr int CB = kChanBlock<MMA_BF16>;
  constexpr int PER = MMA_BF16 ? 8 : 4;           // channels per lane per block
  const Plan& p = a.p;
  const int i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N, d = p.d;

  // W fragments and logistic biases, in registers for the whole wave
  FT wf[NCT][KCH];
  float bdr[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ct + i;
    const bool sc = col < K, zc = col >= K && col < K + N;
    const void* wb = sc ? a.W_sel : a.W_d;
    const size_t wrow = sc ? ((size_t)h * K + col) * d : ((size_t)h * N + (col - K)) * d;
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      const int ch = m * CB + PER * g;
      wf[ct][m] = load_frag<IN_BF16, MMA_BF16>(wb, wrow + ch, (sc || zc) && ch < d);
    }
    bdr[ct] = zc ? a.b_d[(size_t)h * N + col - K] : 0.f;
  }

  const size_t ubase = ((size_t)s_u * p.L + c0) * d;
  FT cur[KCH], nxt[KCH];
  {
    const int row = rbeg + i;
#pragma unroll
    for (int m = 0; m < KCH; ++m)
      cur[m] = load_frag<IN_BF16, MMA_BF16>(a.u, ubase + (size_t)row * d + m * CB + PER * g,
                                            row < rend);
  }
  for (int row0 = rbeg; row0 < rend; row0 += 16) {
    const int nrow = row0 + 16 + i;
#pragma unroll
    for (int m = 0; m < KCH; ++m)
      nxt[m] = load_frag<IN_BF16, MMA_BF16>(a.u, ubase + (size_t)nrow * d + m * CB + PER * g,
                                            nrow < rend);
    f4v acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KCH; ++m)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) mma_step<IN_BF16, MMA_BF16>(acc[ct], cur[m], wf[ct][m]);
    tile_epilogue<NCT>(p, acc, bdr, row0, rend, lane, o);
#pragma unroll
    for (int m = 0; m < KCH; ++m) cur[m] = nxt[m];
  }
}

// Any shape: operands loaded per 16-row tile, up to 8 column tiles.
template <int IN_BF16, int MMA_BF16>
__device__ __forceinline__ void select_rows_any(const Args& a, int s_u, int h, int c0, int rbeg,
                                                int rend, int lane, const SelDst& o) {
  typedef typename Frag<IN_BF16, MMA_BF16>::T FT;
  constexpr int CB = kChanBlock<MMA_BF16>;
  constexpr int PER = MMA_BF16 ? 8 : 4;
  const Plan& p = a.p;
  const int i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N, d = p.d;
  const int NCT = p.NC >> 4;
  float bdr[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int col = 16 * ct + i;
    bdr[ct] = (ct < NCT && col >= K && col < K + N) ? a.b_d[(size_t)h * N + col - K] : 0.f;
  }
  const size_t ubase = ((size_t)s_u * p.L + c0) * d;
  for (int row0 = rbeg; row0 < rend; row0 += 16) {
    const int row = row0 + i;
    f4v acc[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = f4v{0.f, 0.f, 0.f, 0.f};
    for (int m = 0; m * CB < d; ++m) {
      const int ch = m * CB + PER * g;
      const FT av = load_frag<IN_BF16, MMA_BF16>(a.u, ubase + (size_t)row * d + ch,
                                                 row < rend && ch < d);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        if (ct < NCT) {
          const int col = 16 * ct + i;
          const bool sc = col < K, zc = col >= K && col < K + N;
          const void* wb = sc ? a.W_sel : a.W_d;
          const size_t wrow = sc ? ((size_t)h * K + col) * d : ((size_t)h * N + (col - K)) * d;
          const FT bw = load_frag<IN_BF16, MMA_BF16>(wb, wrow + ch, (sc || zc) && ch < d);
          mma_step<IN_BF16, MMA_BF16>(acc[ct], av, bw);
        }
      }
    }
    switch (NCT) {
      case 1: tile_epilogue<1>(p, acc, bdr, row0, rend, lane, o); break;
      case 2: tile_epilogue<2>(p, acc, bdr, row0, rend, lane, o); break;
      case 3: tile_epilogue<3>(p, acc, bdr, row0, rend, lane, o); break;
      case 4: tile_epilogue<4>(p, acc, bdr, row0, rend, lane, o); break;
      case 5: tile_epilogue<5>(p, acc, bdr, row0, rend, lane, o); break;
      case 6: tile_epilogue<6>(p, acc, bdr, row0, rend, lane, o); break;
      case 7: tile_epilogue<7>(p, acc, bdr, row0, rend, lane, o); break;
      default: tile_epilogue<8>(p, acc, bdr, row0, rend, lane, o); break;
    }
  }
}

// Shapes with a register-resident fast path.
enum SelPath : int { kSelAny = 0, kSelF32D64N2 = 1, kSelF32D16N1 = 2, kSelBF16D128N3 = 3 };

template <int IN_BF16, int MMA_BF16, int PATH>
__device__ __forceinline__ void select_dispatch(const Args& a, int s_u, int h, int c0, int rbeg,
                                                int rend, int lane, const SelDst& o) {
  if constexpr (PATH == kSelF32D64N2 && !IN_BF16 && !MMA_BF16)
    select_rows<0, 0, 4, 2>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH == kSelF32D16N1 && !IN_BF16 && !MMA_BF16)
    select_rows<0, 0, 1, 1>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH == kSelBF16D128N3 && IN_BF16 && MMA_BF16)
    select_rows<1, 1, 4, 3>(a, s_u, h, c0, rbeg, rend, lane, o);
  else
    select_rows_any<IN_BF16, MMA_BF16>(a, s_u, h, c0, rbeg, rend, lane, o);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int MODE, int IN_BF16, int MMA_BF16, int PATH>
__device__ __forceinline__ void pdssm_body(const Args& a, unsigned char* smem) {
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, NP = p.NP, S = p.S, T = p.chunk, TS = p.TS;
  const int BH = p.B * p.H;

  float* Dbuf = (float*)(smem + p.off_D);
  int* kbuf = (int*)(smem + p.off_k);
  float* yloc = (float*)(smem + p.off_yl);
  int* dic = (int*)(smem + p.off_dict);
  i2v* DC = (i2v*)(smem + p.off_DC);
  float* Cs = (float*)(smem + p.off_C);
  float* slots = (float*)(smem + p.off_slot);
  int* sIdx = (int*)(smem + p.off_sIdx);
  float* sSc = (float*)(smem + p.off_sSc);
  float* sB = (float*)(smem + p.off_sB);
  int* pIdx = (int*)(smem + p.off_pIdx);
  float* pSc = (float*)(smem + p.off_pSc);
  float* pB = (float*)(smem + p.off_pB);
  float* Hs = (float*)(smem + p.off_H);
  float* tmp = (float*)(smem + p.off_tmp);
  int* misc = (int*)(smem + p.off_misc);

  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* agg = (uint64_t*)(a.ws + p.ws_agg);
  uint64_t* inc = (uint64_t*)(a.ws + p.ws_inc);

  // ---- task: chunk-major tickets so that predecessors always started first
  int task;
  if constexpr (MODE == kModeSelect) {
    task = blockIdx.x;
  } else {
    if (tid == 0) misc[0] = (int)atomicAdd(&hdr[kWsTicket], 1u);
    __syncthreads();
    task = misc[0];
  }
  const int c = task / BH, s = task % BH;
  const int b = s / p.H, h = s % p.H;
  const int c0 = c * T;
  const int Tc = min(T, p.L - c0);
  const size_t gbase = (size_t)s * p.L + c0;

  const int gpw = 64 / NP;                 // lane groups per wave
  const int gl = lane / NP, j = lane % NP;
  const int gam = wave * gpw + gl;         // this lane's group (sub-chunk)
  const int tb = gam * S, te = min(tb + S, Tc);
  const bool act = j < N;

  // ---- phase-A drive terms of the first block: issued first, used last
  float bu[kBuBlock];
  if constexpr (MODE != kModeSelect) {
#pragma unroll
    for (int q = 0; q < kBuBlock; ++q) {
      const int t = tb + q;
      bu[q] = (act && t < te) ? a.Bu[(gbase + t) * N + j] : 0.f;
    }
  }

  // ---- per-head constants
  if constexpr (MODE == kModeSelect) {
    if (a.P_out)
      for (int q = tid; q < K * N; q += kThreads) dic[q] = a.dict[(size_t)h * K * N + q];
  } else {
    for (int q = tid; q < N; q += kThreads) Cs[q] = a.C[(size_t)h * N + q];
    __syncthreads();
    // DC[k][m] = (dict[k][m], C[dict[k][m]]): target row and its output weight
    for (int q = tid; q < K * N; q += kThreads) {
      const int r = a.dict[(size_t)h * K * N + q];
      DC[q] = i2v{r, __float_as_int(Cs[r])};
    }
  }
  if constexpr (MODE == kModeScan) {
    for (int q = tid; q < Tc; q += kThreads) kbuf[q] = a.k_in[gbase + q];
    for (int q = tid; q < Tc * N; q += kThreads) {
      const int t = q / N, n = q - t * N;
      Dbuf[n * TS + t] = a.D_in[gbase * N + q];
    }
  }
  __syncthreads();

  // ---- selection for this wave's rows
  if constexpr (MODE != kModeScan) {
    const int s_u = p.u_shared ? b : s;
    SelDst o;
    o.kbuf = (MODE == kModeFused) ? kbuf : nullptr;
    o.Dbuf = (MODE == kModeFused) ? Dbuf : nullptr;
    o.TS = TS;
    o.k_out = a.k_out;
    o.D_out = a.D_out;
    o.P_out = a.P_out;
    o.dic = dic;
    o.gbase = gbase;
    const int wr0 = min(wave * gpw * S, Tc), wr1 = min(wr0 + gpw * S, Tc);
    select_dispatch<IN_BF16, MMA_BF16, PATH>(a, s_u, h, c0, wr0, wr1, lane, o);
  }
  if constexpr (MODE == kModeSelect) return;
  WAVE_SYNC();   // this wave's k* / D rows are read back by its own lane groups

  // ---- phase A: each lane group runs its sub-chunk [tb, te) from a zero state
  float* slot = slots + gam * NP;
  const float cj = act ? Cs[j] : 0.f;
  float hl = 0.f, msc = 1.f;
  int midx = j;
  for (int blk = 0; blk < S; blk += kBuBlock) {
    if (blk > 0) {
#pragma unroll
      for (int q = 0; q < kBuBlock; ++q) {
        const int t = tb + blk + q;
        bu[q] = (act && t < te) ? a.Bu[(gbase + t) * N + j] : 0.f;
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < kBuBlock; q4 += 4) {
      const int t0 = tb + blk + q4;
      if (blk + q4 >= S) break;               // uniform across the workgroup
      const bool gv0 = t0 < te;               // uniform within the group
      // state-independent inputs of the next four steps
      i4v k4 = {0, 0, 0, 0};
      f4v d4 = {0.f, 0.f, 0.f, 0.f};
      if (gv0) {
        k4 = *(const i4v*)(kbuf + t0);
        if (act) d4 = *(const f4v*)(Dbuf + j * TS + t0);
      }
      int id4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) id4[r] = (act && t0 + r < te) ? DC[k4[r] * N + j].x : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        const bool gv = t < te;
        const bool v = act && gv;
        // the running map's next factor, gathered at its current rows
        i2v e = {0, 0};
        float dm = 0.f;
        if (v) {
          e = DC[k4[r] * N + midx];
          dm = Dbuf[midx * TS + t];
        }
        // h' = Bu + scatter(D h): one wave, so its LDS operations stay in order
        if (v) slot[j] = bu[q4 + r];
        if (v) atomicAdd(&slot[id4[r]], d4[r] * hl);
        if (v) hl = slot[j];
        // compose, and record w_t = C Phi_t over column t (every lane of the
        // group has read column t above)
        if (v) {
          msc *= dm;
          midx = e.x;
          Dbuf[j * TS + t] = __int_as_float(e.y) * msc;
        }
        // local output C h'
        const float yl = group_sum(v ? cj * hl : 0.f, NP);
        if (gv && j == 0) yloc[t] = yl;
      }
    }
  }
  if (act) {
    sIdx[gam * N + j] = midx;
    sSc[gam * N + j] = msc;
    sB[gam * N + j] = hl;
  }
  __syncthreads();

  // ---- combine the sub-chunk summaries in order (wave 0)
  if (wave == 0) {
    const bool on = lane < N;
    int ai = lane;
    float as = 1.f, ab = 0.f;
    for (int gm = 0; gm < p.G; ++gm) {
      int gi = 0;
      float gs = 0.f, gb = 0.f;
      if (on) {
        pIdx[gm * N + lane] = ai;
        pSc[gm * N + lane] = as;
        pB[gm * N + lane] = ab;
        gi = sIdx[gm * N + lane];
        gs = sSc[gm * N + lane];
        gb = sB[gm * N + lane];
      }
      const int ni = on ? sIdx[gm * N + ai] : 0;
      const float ns = on ? sSc[gm * N + ai] * as : 0.f;
      if (on) tmp[lane] = gb;
      WAVE_SYNC();
      if (on) atomicAdd(&tmp[gi], gs * ab);
      WAVE_SYNC();
      if (on) ab = tmp[lane];
      WAVE_SYNC();
      ai = ni;
      as = ns;
    }

    // ---- publish this chunk's aggregate
    uint64_t* my = agg + ((size_t)c * BH + s) * 3 * N;
    if (on) {
      put_tagged(my + lane, (uint32_t)ai);
      put_tagged(my + N + lane, __float_as_uint(as));
      put_tagged(my + 2 * N + lane, __float_as_uint(ab));
    }

    // ---- look back for the carry into this chunk
    float x = (on && a.h0) ? a.h0[(size_t)s * N + lane] : 0.f;
    if (c > 0) {
      int q = c - 1, spins = 0, start = 0;
      while (true) {
        const uint64_t wi = on ? get_tagged(inc + ((size_t)q * BH + s) * N + lane) : kTagValid;
        if (__all(tag_ok(wi))) {
          x = __uint_as_float((uint32_t)wi);
          start = q + 1;
          break;
        }
        uint64_t* pa = agg + ((size_t)q * BH + s) * 3 * N;
        bool okq = true;
        if (on) okq = tag_ok(get_tagged(pa + lane)) && tag_ok(get_tagged(pa + N + lane)) &&
                      tag_ok(get_tagged(pa + 2 * N + lane));
        if (__all(okq)) {
          if (q == 0) { start = 0; break; }  // x holds h0
          --q;
          continue;
        }
        if (++spins > kSpinLimit) {
          if (lane == 0) atomicOr(&hdr[kWsError], 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      for (int r = start; r < c; ++r) {
        uint64_t* pa = agg + ((size_t)r * BH + s) * 3 * N;
        int ri = 0;
        float rs = 0.f, rb = 0.f;
        if (on) {
          ri = (int)(uint32_t)get_tagged(pa + lane);
          rs = __uint_as_float((uint32_t)get_tagged(pa + N + lane));
          rb = __uint_as_float((uint32_t)get_tagged(pa + 2 * N + lane));
        }
        if (on) tmp[lane] = rb;
        WAVE_SYNC();
        if (on) atomicAdd(&tmp[ri], rs * x);
        WAVE_SYNC();
        if (on) x = tmp[lane];
        WAVE_SYNC();
      }
    }
    // inclusive state of this chunk, with the same arithmetic
    if (on) tmp[lane] = ab;
    WAVE_SYNC();
    if (on) atomicAdd(&tmp[ai], as * x);
    WAVE_SYNC();
    const float xo = on ? tmp[lane] : 0.f;
    WAVE_SYNC();
    if (on) {
      put_tagged(inc + ((size_t)c * BH + s) * N + lane, __float_as_uint(xo));
      Hs[lane] = x;
      if (c == p.nC - 1) a.hL[(size_t)s * N + lane] = xo;
    }
  }
  __syncthreads();

  // ---- phase C: carries into every sub-chunk, then the corrected outputs
  {
    const int gm = tid / NP, jj = tid % NP;
    const bool on = jj < N;
    slots[tid] = on ? pB[gm * N + jj] : 0.f;
    __syncthreads();
    if (on) atomicAdd(&slots[gm * NP + pIdx[gm * N + jj]], pSc[gm * N + jj] * Hs[jj]);
    __syncthreads();
  }
  for (int t = tid; t < Tc; t += kThreads) {
    const float* cr = slots + (t / S) * NP;
    float acc = yloc[t];
    for (int n = 0; n < N; ++n) acc += Dbuf[n * TS + t] * cr[n];
    a.y[gbase + t] = acc;
  }
}

// Two entry points over one body: the register-resident fp32 selection paths
// fit three waves per SIMD; the other paths get the larger register budget
// of two waves per SIMD.
template <int MODE, int IN_BF16, int MMA_BF16, int PATH>
__global__ __launch_bounds__(kThreads, 3) void pdssm_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  pdssm_body<MODE, IN_BF16, MMA_BF16, PATH>(a, smem);
}

template <int MODE, int IN_BF16, int MMA_BF16, int PATH>
__global__ __launch_bounds__(kThreads, 2) void pdssm_kernel_wide(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  pdssm_body<MODE, IN_BF16, MMA_BF16, PATH>(a, smem);
}

// Zero the workspace words the scan reads (header, aggregates, inclusive states).
__global__ void clear_kernel(uint64_t* w, size_t n) {
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    w[q] = 0;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static int sel_path(const Plan& p) {
  const int nct = p.NC >> 4;
  if (!p.in_bf16 && p.d == 64 && nct == 2) return kSelF32D64N2;
  if (!p.in_bf16 && p.d == 16 && nct == 1) return kSelF32D16N1;
  if (p.in_bf16 && p.mma_bf16 && p.d == 128 && nct == 3) return kSelBF16D128N3;
  return kSelAny;
}

template <int MODE, int IN_BF16, int MMA_BF16>
static void launch_path(const Args& a, int path, dim3 grid, hipStream_t st) {
  const dim3 block(kThreads);
  const int lds = a.p.lds_bytes;
  switch (path) {
    case kSelF32D64N2:
      hipLaunchKernelGGL((pdssm_kernel<MODE, IN_BF16, MMA_BF16, kSelF32D64N2>), grid, block, lds, st, a);
      break;
    case kSelF32D16N1:
      hipLaunchKernelGGL((pdssm_kernel<MODE, IN_BF16, MMA_BF16, kSelF32D16N1>), grid, block, lds, st, a);
      break;
    case kSelBF16D128N3:
      hipLaunchKernelGGL((pdssm_kernel_wide<MODE, IN_BF16, MMA_BF16, kSelBF16D128N3>), grid, block, lds, st, a);
      break;
    default:
      if (MODE == kModeScan)
        hipLaunchKernelGGL((pdssm_kernel<MODE, IN_BF16, MMA_BF16, kSelAny>), grid, block, lds, st, a);
      else
        hipLaunchKernelGGL((pdssm_kernel_wide<MODE, IN_BF16, MMA_BF16, kSelAny>), grid, block, lds, st, a);
  }
}

template <int MODE>
static hipError_t launch_mode(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  const dim3 grid(p.tasks);
  if (MODE != kModeSelect) {
    const size_t words = p.ws_bytes / 8;
    size_t cb = (words + 255) / 256;
    if (cb > 4096) cb = 4096;
    if (cb < 1) cb = 1;
    hipLaunchKernelGGL(clear_kernel, dim3((unsigned)cb), dim3(256), 0, st, (uint64_t*)a.ws, words);
  }
  if constexpr (MODE == kModeScan) {
    launch_path<MODE, 0, 0>(a, kSelAny, grid, st);   // no selection in this mode
  } else {
    const int path = sel_path(p);
    if (p.in_bf16 && p.mma_bf16) launch_path<MODE, 1, 1>(a, path, grid, st);
    else if (p.in_bf16) launch_path<MODE, 1, 0>(a, path, grid, st);
    else launch_path<MODE, 0, 0>(a, path, grid, st);
  }
  return hipGetLastError();
}

hipError_t launch(int mode, const Args& a, hipStream_t st) {
  switch (mode) {
    case kModeSelect: return launch_mode<kModeSelect>(a, st);
    case kModeScan: return launch_mode<kModeScan>(a, st);
    default: return launch_mode<kModeFused>(a, st);
  }
}

}  // namespace pdscan

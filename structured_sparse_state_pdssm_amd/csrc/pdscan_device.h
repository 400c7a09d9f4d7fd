// Device code for gfx950 (CDNA4): selection, chunked scan, and the fused pass.
// Included by the three launcher translation units (one per mode), which are
// compiled in parallel.
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

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "pdscan_plan.h"

namespace pdscan {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef int i4v __attribute__((ext_vector_type(4)));
typedef int i2v __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr uint64_t kTagValid = 1ull << 32;
constexpr int kBuBlock = 16;   // phase-A steps whose drive terms sit in registers

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

// Raw buffer loads through a per-workgroup resource: a scalar base, 32-bit
// lane offsets, and reads past the end return zero without touching memory
// (kNoLoad is such an offset).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;     // 32-bit data format, raw access
constexpr uint32_t kNoLoad = 0xFFFFFFF0u;

// `base` and `bytes` must be the same in every lane of the wave (every
// descriptor here is per workgroup).  They are taken through lane 0 so the
// descriptor stays in scalar registers even where the compiler cannot prove
// them uniform (values derived from a ticket read back from LDS); a
// descriptor in vector registers turns each load into a loop over lanes.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}
__device__ __forceinline__ float buf_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ int buf_i32(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, n - 1>) in
// order: a loop unrolled by construction, whatever its body's size.
template <class F, int... Ks>
__device__ __forceinline__ void unrolled(std::integer_sequence<int, Ks...>, F&& f) {
  (f(std::integral_constant<int, Ks>{}), ...);
}

// DPP lane permutations inside 16-lane rows.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Every pattern here reads a valid lane; bound_ctrl with a zero "old" lets
// the compiler fold the move into the consuming VALU instruction.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

// Order-preserving integer key of a finite float (-0 folded onto +0, so
// equal scores give equal keys).
__device__ __forceinline__ int order_key(float v) {
  const int b = __float_as_int(v + 0.0f);
  return b ^ ((b >> 31) & 0x7fffffff);
}

// Max / min over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ int row_max(int v) {
  v = max(v, dpp_i<kDppXor1>(v));
  v = max(v, dpp_i<kDppXor2>(v));
  v = max(v, dpp_i<kDppHalfMirror>(v));
  return max(v, dpp_i<kDppMirror>(v));
}
__device__ __forceinline__ int row_min(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  return min(v, dpp_i<kDppMirror>(v));
}

// Apply a map inside one 16-lane DPP row without atomics: lane i returns
// base + sum of v_j over the lanes j of its row whose idx_j == i, visiting
// j = i, i+1, ... (mod 16) in a fixed order.
template <int S>
__device__ __forceinline__ void gather_rot(float& acc, int idx, float v, int i) {
  const int ix = dpp_i<0x120 + S>(idx);      // row_ror:S
  const float vs = dpp_f<0x120 + S>(v);
  acc += (ix == i) ? vs : 0.f;
}
__device__ __forceinline__ float row_gather_add(float base, int idx, float v, int i) {
  float acc = base + ((idx == i) ? v : 0.f);
  gather_rot<1>(acc, idx, v, i);
  gather_rot<2>(acc, idx, v, i);
  gather_rot<3>(acc, idx, v, i);
  gather_rot<4>(acc, idx, v, i);
  gather_rot<5>(acc, idx, v, i);
  gather_rot<6>(acc, idx, v, i);
  gather_rot<7>(acc, idx, v, i);
  gather_rot<8>(acc, idx, v, i);
  gather_rot<9>(acc, idx, v, i);
  gather_rot<10>(acc, idx, v, i);
  gather_rot<11>(acc, idx, v, i);
  gather_rot<12>(acc, idx, v, i);
  gather_rot<13>(acc, idx, v, i);
  gather_rot<14>(acc, idx, v, i);
  gather_rot<15>(acc, idx, v, i);
  return acc;
}

// Sum over a lane group of NP lanes (a power of two); every lane of the group
// gets the same value (the partial sums meet in the same order on every lane).
template <int NP>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (NP >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (NP >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (NP >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (NP >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (NP >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (NP >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Group sums of four values at once (NP = 32 or 64): lane l ends with the
// sum over its group of v[l & 3].  Two exchange levels inside each quad leave
// every lane the quad sum of one value (l & 3), rotations by 4 and 8 finish
// each 16-lane row, and permutes join the rows: 6 or 7 exchanges instead of
// 4 x 6 for four separate sums.  The order of the additions is fixed.
constexpr int kDppRor4 = 0x124;        // row_ror:4
constexpr int kDppRor8 = 0x128;        // row_ror:8
template <int NP>
__device__ __forceinline__ float group_sum4(const float (&v)[4], int lane) {
  static_assert(NP == 32 || NP == 64, "rows joined by permutes");
  const bool o1 = lane & 1, o2 = lane & 2;
  const float a = (o1 ? v[1] : v[0]) + dpp_f<kDppXor1>(o1 ? v[0] : v[1]);
  const float b = (o1 ? v[3] : v[2]) + dpp_f<kDppXor1>(o1 ? v[2] : v[3]);
  float c = (o2 ? b : a) + dpp_f<kDppXor2>(o2 ? a : b);
  c += dpp_f<kDppRor4>(c);
  c += dpp_f<kDppRor8>(c);
  c += __shfl_xor(c, 16, 64);
  if constexpr (NP == 64) c += __shfl_xor(c, 32, 64);
  return c;
}

// The same sum, complete only in the group's last 16-lane row (lanes
// NP - 16 .. NP - 1; NP <= 16: every lane): rows are joined by DPP row
// broadcasts (lane 15 of a row into the next row, lane 31 into rows 2 and 3)
// instead of cross-lane permutes through the LDS unit.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int NP>
__device__ __forceinline__ float group_sum_last(float v) {
  v = group_sum<NP < 16 ? NP : 16>(v);
  if constexpr (NP >= 32)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppRowBcast15,
                                                               0xA, 0xF, false));
  if constexpr (NP >= 64)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppRowBcast31,
                                                               0xC, 0xF, false));
  return v;
}

__device__ __forceinline__ float group_sum_rt(float v, int NP) {
  switch (NP) {
    case 1: return v;
    case 2: return group_sum<2>(v);
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
  }
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
  unsigned char* wst;  // deep path: LDS stages for the weight blocks, or nullptr
  float* Bubuf;   // drive folded: [N][TS] drive terms of the chunk (fused), or nullptr
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
__device__ __forceinline__ typename Frag<IN_BF16, MMA_BF16>::T load_frag_buf(rsrc_t r, uint32_t off) {
  typedef typename Frag<IN_BF16, MMA_BF16>::T T;
  if constexpr (IN_BF16 && !MMA_BF16)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
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

// fp32 products on the bf16 matrix cores.  Truncation splits an fp32 value
// exactly into three bf16 pieces, x = x0 + x1 + x2 (each piece holds the next
// eight significant bits, so each remainder is exact); the six piece products
// with i + j <= 2 are exact in fp32 and are accumulated in fp32, and the
// terms left out are below 2^-23 of |x w|.  This is a standard fp32 GEMM
// emulation; it keeps the scores and pre-activations at fp32 accuracy.
__device__ __forceinline__ unsigned hi16_pair(float lo, float hi) {
  // bf16 pair (lo in the low half) from the high halves of two fp32 words
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ u4v pack_hi8(const f4v& a, const f4v& b) {
  return u4v{hi16_pair(a.x, a.y), hi16_pair(a.z, a.w), hi16_pair(b.x, b.y), hi16_pair(b.z, b.w)};
}
__device__ __forceinline__ f4v trunc_rem(const f4v& a) {
  // a minus its bf16 truncation (exact)
  f4v t;
  t.x = __uint_as_float(__float_as_uint(a.x) & 0xFFFF0000u);
  t.y = __uint_as_float(__float_as_uint(a.y) & 0xFFFF0000u);
  t.z = __uint_as_float(__float_as_uint(a.z) & 0xFFFF0000u);
  t.w = __uint_as_float(__float_as_uint(a.w) & 0xFFFF0000u);
  return a - t;
}
// the three pieces of eight fp32 values (two fragments), as bf16 operands
__device__ __forceinline__ void split3(f4v a, f4v b, u4v* pc) {
  pc[0] = pack_hi8(a, b);
  a = trunc_rem(a);
  b = trunc_rem(b);
  pc[1] = pack_hi8(a, b);
  a = trunc_rem(a);
  b = trunc_rem(b);
  pc[2] = pack_hi8(a, b);
}
// acc += x w over 32 channels, x and w given as three pieces each
__device__ __forceinline__ void mma_split3(f4v& acc, const u4v* x, const u4v* w) {
  auto mm = [&](const u4v& p, const u4v& q) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, p), __builtin_bit_cast(bf8v, q),
                                                  acc, 0, 0, 0);
  };
  mm(x[2], w[0]);                                  // smallest terms first
  mm(x[1], w[1]);
  mm(x[0], w[2]);
  mm(x[1], w[0]);
  mm(x[0], w[1]);
  mm(x[0], w[0]);
}

// channels per fragment block: 16 (fp32 MFMA, 4 per lane group) or 32 (bf16)
template <int MMA_BF16>
constexpr int kChanBlock = MMA_BF16 ? 32 : 16;

// Epilogue of one tile: argmax over score columns, logistic of the
// pre-activations, drive terms (drive folded), stores.  rows >= rlim are not
// stored.  Columns: [0, K) scores, [K, K + N) pre-activations, [K + N,
// K + 2N) drive terms.  Column of tile t: 16 t + i when kt < 0 (the three
// segments contiguous); with kt >= 0 the first kt tiles hold the scores,
// the next ceil(N / 16) the pre-activations (column K + 16 (t - kt) + i) and
// the ones after them the drive terms, so that no tile straddles two weight
// matrices.
template <int NCT>
__device__ __forceinline__ void tile_epilogue(const Plan& p, const f4v* acc, const float* bdr,
                                              int row0, int rlim, int lane, const SelDst& o,
                                              int ct0 = 0, int kt = -1) {
  // ct0: the first column tile held in acc; the score columns (K <= 64, at
  // most four tiles) are always in the pass that starts at 0
  const bool with_k = ct0 == 0;
  const int i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N;
  // argmax per row: the largest score over the row's lanes, then the lowest
  // column holding it (lowest index wins ties)
  int bv[4];
  int bk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    bv[r] = (int)0x80000000;
    bk[r] = 0x7fffffff;
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * (ct0 + ct) + i;
    if (16 * (ct0 + ct) < K) {             // uniform: tile holds score columns
      const bool sc = col < K;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = sc ? order_key(acc[ct][r]) : (int)0x80000000;
        const bool gt = v > bv[r];         // columns rise with ct: keep the first
        bv[r] = gt ? v : bv[r];
        bk[r] = gt ? col : bk[r];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = row_max(bv[r]);
    bk[r] = row_min(bv[r] == m ? bk[r] : 0x7fffffff);
  }
  const int rb = row0 + 4 * g;   // first of this lane's four rows
  const bool full = rb + 4 <= rlim;
  if (with_k && i == 0) {
    if (o.kbuf) {
      if (full) *(i4v*)(o.kbuf + rb) = i4v{bk[0], bk[1], bk[2], bk[3]};
      else
        for (int r = 0; r < 4; ++r) if (rb + r < rlim) o.kbuf[rb + r] = bk[r];
    }
    if (o.k_out)
      for (int r = 0; r < 4; ++r) if (rb + r < rlim) o.k_out[o.gbase + rb + r] = bk[r];
  }
  const int nt = (N + 15) >> 4;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int t = ct0 + ct;
    const int col = (kt < 0 || t < kt) ? 16 * t + i
                                       : (t < kt + nt ? K + 16 * (t - kt) + i : K + N + 16 * (t - kt - nt) + i);
    if (o.Bubuf && col >= K + N && col < K + 2 * N) {
      // drive term Bu_t[n] = W_b[n, :] u_t, raw
      float* dst = o.Bubuf + (col - K - N) * o.TS + rb;
      if (full) *(f4v*)dst = acc[ct];
      else
        for (int r = 0; r < 4; ++r) if (rb + r < rlim) dst[r] = acc[ct][r];
    }
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
  if (with_k && o.P_out) {
    for (int r = 0; r < 4; ++r)
      for (int gg = 0; gg < 4; ++gg) {
        const int kr = __shfl(bk[r], 16 * gg, 64);
        const int row = row0 + 4 * gg + r;
        if (row < rlim)
          for (int n = lane; n < N; n += 64) o.P_out[(o.gbase + row) * N + n] = o.dic[kr * N + n];
      }
  }
}

template <int IN_BF16, int MMA_BF16, int KCH, int NCT, int FOLD>
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
    const bool bc = FOLD && col >= K + N && col < K + 2 * N;   // drive folded: rows of W_b
    const void* wb = sc ? a.W_sel : (zc ? a.W_d : a.W_b);
    const size_t wrow = sc ? ((size_t)h * K + col) * d
                           : (zc ? ((size_t)h * N + (col - K)) * d : ((size_t)h * N + (col - K - N)) * d);
#pragma unroll
    for (int m = 0; m < KCH; ++m) {
      const int ch = m * CB + PER * g;
      wf[ct][m] = load_frag<IN_BF16, MMA_BF16>(wb, wrow + ch, (sc || zc || bc) && ch < d);
    }
    bdr[ct] = zc ? a.b_d[(size_t)h * N + col - K] : 0.f;
  }

  // this chunk's rows of u through one buffer resource (rows past the
  // chunk read as zero)
  constexpr int ES = IN_BF16 ? 2 : 4;
  const int Tc = min(p.chunk, p.L - c0);
  const rsrc_t ur = make_rsrc((const unsigned char*)a.u + ((size_t)s_u * p.L + c0) * d * ES,
                              (uint32_t)(Tc * d * ES));
  // one tile in flight while the previous one is multiplied
  FT r0[KCH], r1[KCH];
  auto load_tile = [&](FT* dst, int row0) {
    const int row = row0 + i;
    const uint32_t rb = row < rend ? (uint32_t)(row * d + PER * g) * ES : kNoLoad;
#pragma unroll
    for (int m = 0; m < KCH; ++m)
      dst[m] = load_frag_buf<IN_BF16, MMA_BF16>(ur, rb == kNoLoad ? kNoLoad : rb + m * CB * ES);
  };
  auto do_tile = [&](const FT* src, int row0) {
    f4v acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KCH; ++m)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) mma_step<IN_BF16, MMA_BF16>(acc[ct], src[m], wf[ct][m]);
    tile_epilogue<NCT>(p, acc, bdr, row0, rend, lane, o);
  };
  load_tile(r0, rbeg);
  for (int row0 = rbeg; row0 < rend; row0 += 32) {
    load_tile(r1, row0 + 16);
    do_tile(r0, row0);
    load_tile(r0, row0 + 32);
    if (row0 + 16 < rend) do_tile(r1, row0 + 16);
  }
}

// Any shape: operands loaded per 16-row tile, up to 8 column tiles.
template <int IN_BF16, int MMA_BF16, int FOLD>
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
          const bool bc = FOLD && col >= K + N && col < K + 2 * N;
          const void* wb = sc ? a.W_sel : (zc ? a.W_d : a.W_b);
          const size_t wrow = sc ? ((size_t)h * K + col) * d
                                 : (zc ? ((size_t)h * N + (col - K)) * d : ((size_t)h * N + (col - K - N)) * d);
          const FT bw = load_frag<IN_BF16, MMA_BF16>(wb, wrow + ch, (sc || zc || bc) && ch < d);
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

// bf16 inputs with a wide contraction (d a multiple of 32, too many weights
// to keep in registers): two 16-row tiles at a time against up to four
// column tiles per pass, with the u and weight fragments of the next two
// 32-channel blocks in flight in a three-slot register ring while the current
// block multiplies.
template <int NCT, int FOLD>
__device__ __forceinline__ void select_rows_deep(const Args& a, int s_u, int h, int c0, int rbeg,
                                                 int rend, int lane, const SelDst& o) {
  const Plan& p = a.p;
  const int i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N, d = p.d;
  const int KB = d >> 5;                           // 32-channel blocks
  // tiles: the first KT hold score columns (rows of W_sel), the rest
  // pre-activation columns (rows of W_d), so that every tile reads one
  // matrix and its loads need no branch (a branch between loads into one
  // register makes the compiler drain every load in flight)
  const int KT = (K + 15) >> 4, NT = (N + 15) >> 4;
  constexpr int CP = NCT <= 6 ? NCT : 4;           // column tiles per pass
  const rsrc_t rs = make_rsrc((const uint16_t*)a.W_sel + (size_t)h * K * d, (uint32_t)(K * d * 2));
  const rsrc_t rz = make_rsrc((const uint16_t*)a.W_d + (size_t)h * N * d, (uint32_t)(N * d * 2));
  // drive folded: tiles KT + NT .. KT + 2 NT - 1 read rows of W_b
  const rsrc_t rbw = make_rsrc(FOLD ? (const uint16_t*)a.W_b + (size_t)h * N * d : nullptr,
                               FOLD ? (uint32_t)(N * d * 2) : 0u);
  const int Tc = min(p.chunk, p.L - c0);
  const rsrc_t ur = make_rsrc((const uint16_t*)a.u + ((size_t)s_u * p.L + c0) * d, (uint32_t)(Tc * d * 2));

  for (int row0 = rbeg; row0 < rend; row0 += 32) {
    uint32_t uoff[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = row0 + 16 * rt + i;
      uoff[rt] = row < rend ? (uint32_t)((row * d + 8 * g) * 2) : kNoLoad;
    }
#pragma unroll
    for (int ct0 = 0; ct0 < NCT; ct0 += CP) {
      // weight rows: tile t < KT reads row 16 t + i of W_sel, tile t >= KT
      // row 16 (t - KT) + i of W_d; the descriptor choice is uniform
      float bdr[CP];
      uint32_t woff[CP];                           // byte offsets (kNoLoad: none)
      rsrc_t wr[CP];
#pragma unroll
      for (int ct = 0; ct < CP; ++ct) {
        const int t = ct0 + ct;
        const int seg = t < KT ? 0 : (t < KT + NT ? 1 : 2);   // W_sel, W_d, W_b
        const int m = seg == 0 ? 16 * t + i : (seg == 1 ? 16 * (t - KT) + i : 16 * (t - KT - NT) + i);
        const bool ok = seg == 0 ? m < K : (seg == 1 ? m < N : (FOLD && t < KT + 2 * NT && m < N));
        woff[ct] = ok ? (uint32_t)((m * d + 8 * g) * 2) : kNoLoad;
        bdr[ct] = (ok && seg == 1) ? a.b_d[(size_t)h * N + m] : 0.f;
        wr[ct] = seg == 0 ? rs : (seg == 1 ? rz : rbw);
      }
      constexpr int RING = CP > 4 ? 2 : 3;         // blocks in flight
      u4v Ar[RING][2], Br[RING][CP];
      auto issue = [&](int slot_m, u4v* A2, u4v* Bn) {
        const bool ok = slot_m < KB;
        const uint32_t mo = (uint32_t)(slot_m * 64);   // 32 channels of bf16
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          A2[rt] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                               ur, (ok && uoff[rt] != kNoLoad) ? uoff[rt] + mo : kNoLoad, 0, 0));
#pragma unroll
        for (int ct = 0; ct < CP; ++ct)
          Bn[ct] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                               wr[ct], (ok && woff[ct] != kNoLoad) ? woff[ct] + mo : kNoLoad, 0, 0));
      };
      f4v acc[2][CP];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CP; ++ct) acc[rt][ct] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < RING - 1; ++q) issue(q, Ar[q], Br[q]);
      // Every block of the ring is multiplied unconditionally: a block past
      // the end was loaded as zeros and adds nothing.  (A product under a
      // condition lets the compiler move its loads into the branch, next to
      // their use, which leaves no load in flight while the others compute.)
      for (int mb = 0; mb < KB; mb += RING) {
#pragma unroll
        for (int q = 0; q < RING; ++q) {
          issue(mb + q + RING - 1, Ar[(q + RING - 1) % RING], Br[(q + RING - 1) % RING]);
          __builtin_amdgcn_sched_barrier(0);       // the loads stay ahead of the products
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < CP; ++ct)
              acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf8v, Ar[q][rt]), __builtin_bit_cast(bf8v, Br[q][ct]), acc[rt][ct], 0, 0, 0);
        }
      }
      tile_epilogue<CP>(p, acc[0], bdr, row0, rend, lane, o, ct0, KT);
      if (row0 + 16 < rend) tile_epilogue<CP>(p, acc[1], bdr, row0 + 16, rend, lane, o, ct0, KT);
    }
  }
}

// The deep path with the weight blocks staged through LDS: each 32-channel
// block of the score and pre-activation weights is read from memory once per
// workgroup, each wave loading one or two of its 16-column tiles, instead
// of once per wave.  Every wave of the workgroup takes part whatever its rows
// (rows past rend load zeros and store nothing), with one barrier per block.
// One pass (NCT <= 6), at most 32 rows per wave.  The two stages hold 16 NCT
// columns of 64 bytes each, at a stride of 80 bytes so that the 16 lanes of a
// fragment read hit distinct banks.  They lie in the region D is written to
// afterwards, so a barrier separates their last read from the epilogues.
// u blocks are loaded three ahead into registers, weight blocks two ahead into
// registers and then one ahead into a stage.
template <int NCT, int FOLD>
__device__ __forceinline__ void select_rows_deep_lds(const Args& a, int s_u, int h, int c0, int rbeg,
                                                     int rend, int lane, const SelDst& o) {
  const Plan& p = a.p;
  // the wave index through lane 0: the descriptor and branch choices below
  // are then scalar (a descriptor the compiler cannot prove uniform turns a
  // load into a loop over lanes)
  const int i = lane & 15, g = lane >> 4, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int K = p.K, N = p.N, d = p.d;
  const int KB = d >> 5;
  const int KT = (K + 15) >> 4, NT = (N + 15) >> 4;
  constexpr int kRow = 80, kStage = 16 * NCT * kRow;
  constexpr int TPW = (NCT + kWaves - 1) / kWaves;   // tiles this wave stages
  unsigned char* wst = o.wst;
  const rsrc_t rs = make_rsrc((const uint16_t*)a.W_sel + (size_t)h * K * d, (uint32_t)(K * d * 2));
  const rsrc_t rz = make_rsrc((const uint16_t*)a.W_d + (size_t)h * N * d, (uint32_t)(N * d * 2));
  const rsrc_t rbw = make_rsrc(FOLD ? (const uint16_t*)a.W_b + (size_t)h * N * d : nullptr,
                               FOLD ? (uint32_t)(N * d * 2) : 0u);
  const int Tc = min(p.chunk, p.L - c0);
  const rsrc_t ur = make_rsrc((const uint16_t*)a.u + ((size_t)s_u * p.L + c0) * d, (uint32_t)(Tc * d * 2));

  uint32_t uoff[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rbeg + 16 * rt + i;
    uoff[rt] = row < rend ? (uint32_t)((row * d + 8 * g) * 2) : kNoLoad;
  }
  // tile t < KT: row 16 t + i of W_sel; KT <= t < KT + NT: row 16 (t - KT) + i
  // of W_d; after them (drive folded) row 16 (t - KT - NT) + i of W_b
  uint32_t toff[TPW];
  int tlds[TPW];
  rsrc_t tr[TPW];
#pragma unroll
  for (int w = 0; w < TPW; ++w) {
    const int t = wave + kWaves * w;               // uniform in the wave
    const int seg = t < KT ? 0 : (t < KT + NT ? 1 : 2);
    const int m = seg == 0 ? 16 * t + i : (seg == 1 ? 16 * (t - KT) + i : 16 * (t - KT - NT) + i);
    const bool ok = t < NCT && (seg == 0 ? m < K : (seg == 1 ? m < N : (FOLD && t < KT + 2 * NT && m < N)));
    toff[w] = ok ? (uint32_t)((m * d + 8 * g) * 2) : kNoLoad;
    tr[w] = seg == 0 ? rs : (seg == 1 ? rz : rbw);
    tlds[w] = (16 * t + i) * kRow + 16 * g;
  }
  float bdr[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int n = 16 * (ct - KT) + i;
    bdr[ct] = (ct >= KT && ct < KT + NT && n < N) ? a.b_d[(size_t)h * N + n] : 0.f;
  }

  u4v Ar[4][2], Wr[2][TPW];
  auto load_u = [&](int m, u4v* A2) {
    const bool ok = m < KB;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      A2[rt] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                           ur, (ok && uoff[rt] != kNoLoad) ? uoff[rt] + (uint32_t)m * 64u : kNoLoad, 0, 0));
  };
  auto load_w = [&](int m, u4v* W) {
    const bool ok = m < KB;
#pragma unroll
    for (int w = 0; w < TPW; ++w)
      W[w] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                          tr[w], (ok && toff[w] != kNoLoad) ? toff[w] + (uint32_t)m * 64u : kNoLoad, 0, 0));
  };
  auto put_w = [&](int m, const u4v* W) {
    unsigned char* st = wst + (m & 1) * kStage;
#pragma unroll
    for (int w = 0; w < TPW; ++w)
      if (wave + kWaves * w < NCT) *(u4v*)(st + tlds[w]) = W[w];
  };

  f4v acc[2][NCT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f4v{0.f, 0.f, 0.f, 0.f};
  load_u(0, Ar[0]);
  load_u(1, Ar[1]);
  load_u(2, Ar[2]);
  load_w(0, Wr[0]);
  load_w(1, Wr[1]);
  put_w(0, Wr[0]);
  load_w(2, Wr[0]);
  // blocks past the end load zeros, stage zeros and add nothing (u blocks
  // three ahead in a four-slot ring)
  for (int m0 = 0; m0 < KB; m0 += 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + q;
      __syncthreads();                             // stage m written; stage m - 1 read by every wave
      load_u(m + 3, Ar[(q + 3) & 3]);
      put_w(m + 1, Wr[(q + 1) & 1]);
      load_w(m + 3, Wr[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);           // the loads stay ahead of the products
      const unsigned char* st = wst + (m & 1) * kStage;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const u4v bf = *(const u4v*)(st + (16 * ct + i) * kRow + 16 * g);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf8v, Ar[q & 3][rt]), __builtin_bit_cast(bf8v, bf), acc[rt][ct], 0, 0, 0);
      }
    }
  }
  __syncthreads();                                 // the stages are D's region from here
  tile_epilogue<NCT>(p, acc[0], bdr, rbeg, rend, lane, o, 0, KT);
  tile_epilogue<NCT>(p, acc[1], bdr, rbeg + 16, rend, lane, o, 0, KT);
}

// The deep path with 64-channel blocks (unfolded, at most six column tiles,
// d a multiple of 64; chosen when its stages fit D's region).  A 32-channel
// block reads half of each 128-byte line of u and of the weights, and the
// other half, read one block later, has often left the L1 by then: on the
// LM-layer shape about 40 % of those lines crossed from L2 twice.  Here each
// block reads whole lines, with half as many blocks and barriers.  u is one
// block ahead in a two-slot ring; weight blocks are two ahead in registers,
// then one ahead in a stage of 16 NCT columns x 128 bytes at a 144-byte
// stride (the same bank spread as the 80-byte stride of the 32-channel
// stages).
template <int NCT>
__device__ __forceinline__ void select_rows_deep_lds64(const Args& a, int s_u, int h, int c0, int rbeg,
                                                       int rend, int lane, const SelDst& o) {
  const Plan& p = a.p;
  const int i = lane & 15, g = lane >> 4, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int K = p.K, N = p.N, d = p.d;
  const int KB = d >> 6;                           // 64-channel blocks
  const int KT = (K + 15) >> 4, NT = (N + 15) >> 4;
  constexpr int kRow = 144, kStage = 16 * NCT * kRow;
  constexpr int TPW = (NCT + kWaves - 1) / kWaves;   // tiles this wave stages
  unsigned char* wst = o.wst;
  const rsrc_t rs = make_rsrc((const uint16_t*)a.W_sel + (size_t)h * K * d, (uint32_t)(K * d * 2));
  const rsrc_t rz = make_rsrc((const uint16_t*)a.W_d + (size_t)h * N * d, (uint32_t)(N * d * 2));
  const int Tc = min(p.chunk, p.L - c0);
  const rsrc_t ur = make_rsrc((const uint16_t*)a.u + ((size_t)s_u * p.L + c0) * d, (uint32_t)(Tc * d * 2));

  uint32_t uoff[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rbeg + 16 * rt + i;
    uoff[rt] = row < rend ? (uint32_t)((row * d + 8 * g) * 2) : kNoLoad;
  }
  // tile t < KT: row 16 t + i of W_sel; KT <= t < KT + NT: row 16 (t - KT) + i of W_d
  uint32_t toff[TPW];
  int tlds[TPW];
  rsrc_t tr[TPW];
#pragma unroll
  for (int w = 0; w < TPW; ++w) {
    const int t = wave + kWaves * w;               // uniform in the wave
    const bool sc = t < KT;
    const int m = sc ? 16 * t + i : 16 * (t - KT) + i;
    const bool ok = t < NCT && (sc ? m < K : (t < KT + NT && m < N));
    toff[w] = ok ? (uint32_t)((m * d + 8 * g) * 2) : kNoLoad;
    tr[w] = sc ? rs : rz;
    tlds[w] = (16 * t + i) * kRow + 16 * g;
  }
  float bdr[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int n = 16 * (ct - KT) + i;
    bdr[ct] = (ct >= KT && ct < KT + NT && n < N) ? a.b_d[(size_t)h * N + n] : 0.f;
  }

  u4v Ar[2][2][2], Wr[2][TPW][2];                  // [slot][row tile or column tile][32-channel half]
  auto load_u = [&](int m, u4v (*A)[2]) {
    const bool ok = m < KB;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        A[rt][hf] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
            ur, (ok && uoff[rt] != kNoLoad) ? uoff[rt] + (uint32_t)m * 128u + 64u * hf : kNoLoad, 0, 0));
  };
  auto load_w = [&](int m, u4v (*W)[2]) {
    const bool ok = m < KB;
#pragma unroll
    for (int w = 0; w < TPW; ++w)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        W[w][hf] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
            tr[w], (ok && toff[w] != kNoLoad) ? toff[w] + (uint32_t)m * 128u + 64u * hf : kNoLoad, 0, 0));
  };
  auto put_w = [&](int m, const u4v (*W)[2]) {
    unsigned char* st = wst + (m & 1) * kStage;
#pragma unroll
    for (int w = 0; w < TPW; ++w)
      if (wave + kWaves * w < NCT) {
        *(u4v*)(st + tlds[w]) = W[w][0];
        *(u4v*)(st + tlds[w] + 64) = W[w][1];
      }
  };

  f4v acc[2][NCT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = f4v{0.f, 0.f, 0.f, 0.f};
  load_u(0, Ar[0]);
  load_w(0, Wr[0]);
  load_w(1, Wr[1]);
  put_w(0, Wr[0]);
  load_w(2, Wr[0]);
  // blocks past the end load zeros, stage zeros and add nothing
  for (int m0 = 0; m0 < KB; m0 += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int m = m0 + q;
      __syncthreads();                             // stage m written; stage m - 1 read by every wave
      load_u(m + 1, Ar[(q + 1) & 1]);
      put_w(m + 1, Wr[(q + 1) & 1]);
      load_w(m + 3, Wr[(q + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);           // the loads stay ahead of the products
      const unsigned char* st = wst + (m & 1) * kStage;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const u4v bf = *(const u4v*)(st + (16 * ct + i) * kRow + 16 * g + 64 * hf);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf8v, Ar[q & 1][rt][hf]), __builtin_bit_cast(bf8v, bf), acc[rt][ct], 0, 0, 0);
        }
    }
  }
  __syncthreads();                                 // the stages are D's region from here
  tile_epilogue<NCT>(p, acc[0], bdr, rbeg, rend, lane, o, 0, KT);
  tile_epilogue<NCT>(p, acc[1], bdr, rbeg + 16, rend, lane, o, 0, KT);
}

// Shapes with a register-resident fast path.
// kSelDeep + n: the deep bf16 path with n column tiles, ceil(K / 16) score
// tiles then ceil(N / 16) pre-activation tiles, rounded up to even (a shape
// with fewer real column tiles computes zero tiles that are never written).
enum SelPath : int {
  kSelAny = 0, kSelF32D64N2 = 1, kSelF32D16N1 = 2, kSelBF16D128N3 = 3, kSelBF16D128N5 = 4, kSelStep32 = 5,
  kSelDeep = 16
};

template <int IN_BF16, int MMA_BF16, int PATH, int FOLD = 0>
__device__ __forceinline__ void select_dispatch(const Args& a, int s_u, int h, int c0, int rbeg,
                                                int rend, int lane, const SelDst& o) {
  if constexpr (PATH == kSelF32D64N2 && !IN_BF16 && !MMA_BF16)
    select_rows<0, 0, 4, 2, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH == kSelF32D16N1 && !IN_BF16 && !MMA_BF16)
    select_rows<0, 0, 1, 1, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH == kSelBF16D128N3 && IN_BF16 && MMA_BF16)
    select_rows<1, 1, 4, 3, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH == kSelBF16D128N5 && IN_BF16 && MMA_BF16)
    select_rows<1, 1, 4, 5, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
  else if constexpr (PATH > kSelDeep && IN_BF16 && MMA_BF16) {
    if constexpr (PATH - kSelDeep <= kFoldMaxTiles) {
      if (o.wst) {
        if constexpr (!FOLD && PATH - kSelDeep <= 6) {
          if (a.p.wst == 2) {                      // 64-channel stages fit
            select_rows_deep_lds64<PATH - kSelDeep>(a, s_u, h, c0, rbeg, rend, lane, o);
            return;
          }
        }
        select_rows_deep_lds<PATH - kSelDeep, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
        return;
      }
    }
    select_rows_deep<PATH - kSelDeep, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
  }
  else
    select_rows_any<IN_BF16, MMA_BF16, FOLD>(a, s_u, h, c0, rbeg, rend, lane, o);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Everything after phase A, shared by the scan bodies: combine the sub-chunk
// summaries, phase B (publish, look back, publish), phase C.  Each lane
// brings the summary (midx, msc, hl) of its group's sub-chunk; w_t is in the
// [N][TS] buffer and the local outputs in yloc.
// ---------------------------------------------------------------------------
// Previous chunks whose states and aggregates phase B reads in one batch, at
// most (the combine's scratch bounds it: 11 chunks at N = 16, 5 at N = 32,
// 2 at N = 64).
constexpr int kLookWin = 16;

template <bool ROW16>
__device__ __forceinline__ void chunk_tail(const Args& a, unsigned char* smem, int c, int s, int Tc,
                                           size_t gbase, int NP, int gam, int j, bool act,
                                           int midx, float msc, float hl) {
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, S = p.S, TS = p.TS, G = p.G;
  const int BH = p.B * p.H;
  float* Dbuf = (float*)(smem + p.off_D);
  float* yloc = (float*)(smem + p.off_yl);
  float* slots = (float*)(smem + p.off_slot);
  int* sIdx = (int*)(smem + p.off_sIdx);
  float* sSc = (float*)(smem + p.off_sSc);
  float* sB = (float*)(smem + p.off_sB);
  int* pIdx = (int*)(smem + p.off_pIdx);
  float* pSc = (float*)(smem + p.off_pSc);
  float* pB = (float*)(smem + p.off_pB);
  float* Hs = (float*)(smem + p.off_H);
  float* tmp = (float*)(smem + p.off_tmp);
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* agg = (uint64_t*)(a.ws + p.ws_agg);
  uint64_t* inc = (uint64_t*)(a.ws + p.ws_inc);
  float* slot = slots + gam * NP;

  // ---- combine the sub-chunk summaries: inclusive prefix over the groups
  // (Hillis-Steele), each step composing with the summary `o` groups back
  int ci = midx;
  float cs = msc, cb = hl;
  for (int o = 1; o < G; o <<= 1) {
    if (act) {
      sIdx[gam * N + j] = ci;
      sSc[gam * N + j] = cs;
      sB[gam * N + j] = cb;
    }
    __syncthreads();
    const bool up = act && gam >= o;
    int ni = 0;
    float ns = 0.f, pb = 0.f;
    if (up) {
      const int q = (gam - o) * N + j;
      const int pi = sIdx[q];
      pb = sB[q];
      ni = sIdx[gam * N + pi];
      ns = sSc[gam * N + pi] * sSc[q];
    }
    if constexpr (ROW16) {
      // 16-lane groups: apply the map by a DPP gather inside the row
      const float nb = row_gather_add(cb, up ? ci : -1, up ? cs * pb : 0.f, j);
      __syncthreads();
      if (up) {
        cb = nb;
        ci = ni;
        cs = ns;
      }
    } else {
      if (act) slot[j] = cb;
      __syncthreads();
      if (up) atomicAdd(&slot[ci], cs * pb);
      __syncthreads();
      if (up) {
        cb = slot[j];
        ci = ni;
        cs = ns;
      }
    }
  }
  if (act) {
    pIdx[gam * N + j] = ci;
    pSc[gam * N + j] = cs;
    pB[gam * N + j] = cb;
  }
  __syncthreads();

  // ---- phase B: publish the chunk aggregate (wave 0); all lanes (NP per
  // chunk) read the inclusive states and aggregates of the previous chunks
  // in one batch into the combine's scratch (free by now).  The nearest
  // inclusive state with every aggregate after it present gives the carry;
  // without one the window is read again (chunk c-1 publishes its state
  // without waiting for this chunk, so the loop ends).
  const int lq = (G - 1) * N + (lane < N ? lane : 0);
  if (wave == 0 && lane < N) {
    uint64_t* my = agg + ((size_t)c * BH + s) * 3 * N;
    put_tagged(my + lane, (uint32_t)pIdx[lq]);
    put_tagged(my + N + lane, __float_as_uint(pSc[lq]));
    put_tagged(my + 2 * N + lane, __float_as_uint(pB[lq]));
  }
  // window rows that fit the scratch (four [wst][N] arrays, then the flags;
  // at least one row for every supported N)
  const int wst = min(kLookWin, ((p.off_pIdx - p.off_sIdx) - 4 * kLookWin) / (16 * N));
  const int wq = min(min(kThreads / NP, wst), c);
  int* wIdx = sIdx;                                // [wst][N] window aggregates and states
  float* wSc = (float*)(wIdx + wst * N);
  float* wB = wSc + wst * N;
  float* wI = wB + wst * N;
  int* wFlag = (int*)(wI + wst * N);               // bit 0: state complete, bit 1: aggregate complete
  int hit = -1;
  for (int spins = 0; wq > 0; ++spins) {
    const int qq = tid / NP, jj = tid % NP;
    const bool in = qq < wq, on = in && jj < N;
    uint64_t iv = kTagValid, m0 = kTagValid, m1 = kTagValid, m2 = kTagValid;
    if (on) {
      const size_t cq = (size_t)(c - 1 - qq) * BH + s;
      iv = get_tagged(inc + cq * N + jj);
      m0 = get_tagged(agg + cq * 3 * N + jj);
      m1 = get_tagged(agg + cq * 3 * N + N + jj);
      m2 = get_tagged(agg + cq * 3 * N + 2 * N + jj);
      wI[qq * N + jj] = __uint_as_float((uint32_t)iv);
      wIdx[qq * N + jj] = (int)(uint32_t)m0;
      wSc[qq * N + jj] = __uint_as_float((uint32_t)m1);
      wB[qq * N + jj] = __uint_as_float((uint32_t)m2);
    }
    const uint64_t bi = __ballot(tag_ok(iv));
    const uint64_t ba = __ballot(tag_ok(m0) && tag_ok(m1) && tag_ok(m2));
    if (in && jj == 0) {                           // NP <= 64: a chunk's lanes share a wave
      const uint64_t gm = NP >= 64 ? ~0ull : (((1ull << NP) - 1ull) << lane);
      wFlag[qq] = ((bi & gm) == gm ? 1 : 0) | ((ba & gm) == gm ? 2 : 0);
    }
    __syncthreads();
    for (int q = 0; q < wq; ++q) {                 // the same answer in every lane
      const int f = wFlag[q];
      if (f & 1) { hit = q; break; }
      if (!(f & 2)) break;
    }
    if (hit >= 0 && !p.force_giveup) break;
    if (spins >= p.spin_limit) {                   // give up: carry h0, flag the call
      hit = -1;
      if (tid == 0) atomicOr(&hdr[kWsError], 1u);
      break;
    }
    __syncthreads();                               // the window is rewritten
    __builtin_amdgcn_s_sleep(1);
  }

  // the carry into this chunk, then the inclusive state (wave 0)
  if (wave == 0) {
    const bool on = lane < N;
    const int ai = pIdx[lq];
    const float as = pSc[lq], ab = pB[lq];
    // x <- scatter of (scale .* x) by idx, plus b: one aggregate applied
    auto apply = [&](float& x, int ri, float rsc, float rb) {
      const float rv = on ? rsc * x : 0.f;
      if constexpr (ROW16) {
        const float xn = row_gather_add(on ? rb : 0.f, on ? ri : -1, rv, lane);
        if (on) x = xn;
      } else {
        if (on) tmp[lane] = rb;
        WAVE_SYNC();
        if (on) atomicAdd(&tmp[ri], rv);
        WAVE_SYNC();
        if (on) x = tmp[lane];
        WAVE_SYNC();
      }
    };
    float x = (on && a.h0) ? a.h0[(size_t)s * N + lane] : 0.f;
    if (hit >= 0) {
      // the inclusive state of chunk c-1-hit, then the aggregates of chunks
      // c-hit .. c-1, oldest first
      if (on) x = wI[hit * N + lane];
      for (int q = hit - 1; q >= 0; --q)
        apply(x, on ? wIdx[q * N + lane] : 0, on ? wSc[q * N + lane] : 0.f, on ? wB[q * N + lane] : 0.f);
    }
    // inclusive state of this chunk, with the same arithmetic
    float xo;
    if constexpr (ROW16) {
      xo = row_gather_add(ab, on ? ai : -1, on ? as * x : 0.f, lane);
    } else {
      if (on) tmp[lane] = ab;
      WAVE_SYNC();
      if (on) atomicAdd(&tmp[ai], as * x);
      WAVE_SYNC();
      xo = on ? tmp[lane] : 0.f;
      WAVE_SYNC();
    }
    if (on) {
      put_tagged(inc + ((size_t)c * BH + s) * N + lane, __float_as_uint(xo));
      Hs[lane] = x;
      if (c == p.nC - 1) a.hL[(size_t)s * N + lane] = xo;
    }
  }
  __syncthreads();

  // ---- phase C: state entering every sub-chunk (apply the inclusive prefix
  // of the groups before it to the carry), then the corrected outputs
  {
    float* srow = slots + gam * NP;
    if constexpr (ROW16) {
      const bool on = act && gam > 0;
      const int q = (gam - 1) * N + j;
      const float hj = act ? Hs[j] : 0.f;
      const float cv = row_gather_add(on ? pB[q] : hj, on ? pIdx[q] : -1,
                                      on ? pSc[q] * hj : 0.f, j);
      if (act) srow[j] = cv;
      __syncthreads();
    } else {
      if (gam == 0) {
        if (act) srow[j] = Hs[j];
      } else if (act) {
        srow[j] = pB[(gam - 1) * N + j];
      }
      __syncthreads();
      if (gam > 0 && act) atomicAdd(&srow[pIdx[(gam - 1) * N + j]], pSc[(gam - 1) * N + j] * Hs[j]);
      __syncthreads();
    }
  }
  if constexpr (!ROW16) {
    if (a.H_all) {
      // The state after every step is wanted as well: each group replays its
      // sub-chunk from the state entering it (the step of phase A, now from
      // the true state), writing the states and the outputs directly.
      const int* kbuf = (const int*)(smem + p.off_k);
      const unsigned char* DR = smem + p.off_DC;
      const float* Cs = (const float*)(smem + p.off_C);
      float* scr = (float*)sIdx + gam * NP;        // free since phase B
      float hj = act ? slots[gam * NP + j] : 0.f;
      const int tb = gam * S, te = min(tb + S, Tc);
      for (int t = tb; t < te; ++t) {
        const size_t row = (gbase + t) * N;
        const int r = act ? (int)DR[kbuf[t] * p.DCS + j] : j;
        const float dj = act ? a.D_in[row + j] : 0.f;
        scr[j] = act ? a.Bu[row + j] : 0.f;
        // one wave holds the group, so its LDS operations stay in order
        atomicAdd(&scr[r], dj * hj);
        hj = scr[j];
        if (act) a.H_all[row + j] = hj;
        const float yl = group_sum_rt(act ? Cs[j] * hj : 0.f, NP);
        if (j == 0) a.y[gbase + t] = yl;
      }
      return;
    }
  }
  const int P = p.n_out;
  if (P == 1) {
    for (int t = tid; t < Tc; t += kThreads) {
      const int gt = t / S;
      const int col = t + (p.skew ? gt : 0);
      const float* cr = slots + gt * NP;
      float acc = yloc[col];
      for (int n = 0; n < N; ++n) acc += Dbuf[n * TS + col] * cr[n];
      a.y[gbase + t] = acc;
    }
  } else {
    // several rows of C: output o of step t at y[(gbase + t) P + o]
    for (int e = tid; e < Tc * P; e += kThreads) {
      const int t = e / P, o = e - t * P;
      const int gt = t / S;
      const int col = t + (p.skew ? gt : 0);
      const float* cr = slots + gt * NP;
      const float* wo = Dbuf + o * N * TS;
      float acc = yloc[o * p.YS + col];
      for (int n = 0; n < N; ++n) acc += wo[n * TS + col] * cr[n];
      a.y[(gbase + t) * P + o] = acc;
    }
  }
}

// Inverse dictionary rows for the general kernel's groups of NG = 32 or 64
// rows.  Entry (k, i) lists the sources j of row i under entry k
// (dict[k][j] = i) in ascending order: the first eight as lane byte offsets
// 4 j with bit 0 set (x: sources 1-4, y: 5-8; an empty byte means no
// source), and bit 25 of y set when the row has more than eight.  One lane
// per entry; a wave covers 64 / NG entries, and lane i of an entry builds
// row i from ballots of its sources' target bits (the loop over entries must
// be uniform in the wave: q = 64 w + lane).
template <int NG>
__device__ __forceinline__ i2v row_entry(int tg, bool on, int q, int lane) {
  // lane = q % 64 holds target tg = dict[k][j] of source j = q % NG under
  // entry k = q / NG, and builds row i = q % NG of the same entry
  constexpr int LB = NG == 32 ? 5 : 6;
  const int i = q & (NG - 1);
  uint64_t m = __builtin_amdgcn_ballot_w64(on);
  if constexpr (NG == 32) m &= (lane & 32) ? 0xFFFFFFFF00000000ull : 0xFFFFFFFFull;
#pragma unroll
  for (int b = 0; b < LB; ++b) {
    const uint64_t bb = __builtin_amdgcn_ballot_w64(on && ((tg >> b) & 1));
    m &= ((i >> b) & 1) ? bb : ~bb;
  }
  const int deg = __builtin_popcountll(m);
  unsigned x = 0, y = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const unsigned s = m ? (unsigned)__builtin_ctzll(m) : 0u;
    const unsigned byt = m ? ((s & (unsigned)(NG - 1)) << 2) | 1u : 0u;
    if (r < 4) x |= byt << (8 * r);
    else y |= byt << (8 * (r - 4));
    m &= m - 1;
  }
  if (deg > 8) y |= 2u << 24;
  return i2v{(int)x, (int)y};
}

// Sum over four sources of one row: sx holds four source bytes (lane byte
// offset 4 j with the presence bit 0 set, the group's lane-0 offset ORed into
// bit 7), vj the value of lane j of the group.  The permute selects its lane
// from address bits 2 to 7 alone (checked on gfx950), so byte m of sx needs
// only a shift, and the presence bits become weights 1.0 / 0.0 through
// byte-to-float conversions, and fma(g, 1, h) = h + g, fma(g, 0, h) = h, so
// the sum equals the selected additions in source order.
// pm is the presence mask 0x01010101 from the plan, opaque to the compiler:
// with a literal it knows that each masked byte is 0 or 1 and extracts the bit
// before converting (two instructions per weight instead of one
// v_cvt_f32_ubyteN).
__device__ __forceinline__ float gather4w(unsigned sx, int vj, float hn, unsigned pm) {
  float g[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    g[m] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(sx >> (8 * m)), vj));
  const unsigned wb = sx & pm;
#pragma unroll
  for (int m = 0; m < 4; ++m) hn = __builtin_fmaf(g[m], (float)((wb >> (8 * m)) & 0xFFu), hn);
  return hn;
}

// k* of four steps at once (key r of each lane = score column i of step r;
// keys past K hold the minimum): the row maximum, then the lowest column that
// reaches it, each level applied to all four steps before the next so that
// the DPP reads never wait on the instruction just before them.
__device__ __forceinline__ void row_argmax4(const int (&key)[4], int i, int (&ks)[4]) {
  int m[4], c[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) m[r] = max(key[r], dpp_i<kDppXor1>(key[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) m[r] = max(m[r], dpp_i<kDppXor2>(m[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) m[r] = max(m[r], dpp_i<kDppHalfMirror>(m[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) m[r] = max(m[r], dpp_i<kDppMirror>(m[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = key[r] == m[r] ? i : 0x7fffffff;
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = min(c[r], dpp_i<kDppXor1>(c[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = min(c[r], dpp_i<kDppXor2>(c[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = min(c[r], dpp_i<kDppHalfMirror>(c[r]));
#pragma unroll
  for (int r = 0; r < 4; ++r) ks[r] = min(c[r], dpp_i<kDppMirror>(c[r]));
}

// NOUT: rows of C the instantiation handles (1, or kMaxOut for the
// multi-output plans, which take p.n_out of them).
template <int MODE, int IN_BF16, int MMA_BF16, int PATH, int NPT, int NOUT = 1, int FOLD = 0>
__device__ __forceinline__ void pdssm_body(const Args& a, unsigned char* smem) {
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, S = p.S, T = p.chunk, TS = p.TS;
  // NPT != 0: compile-time group width equal to N (every lane owns a row)
  const int NP = NPT ? NPT : p.NP;
  const int BH = p.B * p.H;

  float* Dbuf = (float*)(smem + p.off_D);
  int* kbuf = (int*)(smem + p.off_k);
  float* yloc = (float*)(smem + p.off_yl);
  int* dic = (int*)(smem + p.off_dict);
  unsigned char* DR = smem + p.off_DC;       // DR[k][m] = dict[k][m] (a byte: N <= 64)
  float* Cs = (float*)(smem + p.off_C);            // row o of C at N o
  float* slots = (float*)(smem + p.off_slot);
  int* misc = (int*)(smem + p.off_misc);
  uint32_t* hdr = (uint32_t*)a.ws;
  // drive folded (fused mode): the selection writes the drive terms here
  // (FOLD: the instantiation for plans with fold_bu set)
  constexpr bool fold = MODE == kModeFused && FOLD;
  float* Bubuf = (float*)(smem + p.off_Bu);
  const int P = NOUT > 1 ? p.n_out : 1;           // rows of C (outputs per step)

  // ---- task: chunk-major tickets so that predecessors always started first
  // (with the die grouping, tickets of this die's class: see xcd_head_groups)
  int c, s;
  if constexpr (MODE == kModeSelect) {
    c = blockIdx.x / BH;
    s = blockIdx.x % BH;
  } else {
    const int hg = p.xhg, cls = blockIdx.x & (kXcds - 1);
    if (tid == 0) misc[0] = (int)atomicAdd(&hdr[hg ? kWsClassTicket + cls : kWsTicket], 1u);
    __syncthreads();
    const int task = misc[0];
    if (hg) {
      const int bg = kXcds / hg, hgi = cls % hg, bgi = cls / hg;
      const int hlo = p.H * hgi / hg, nh = p.H * (hgi + 1) / hg - hlo;
      const int blo = p.B * bgi / bg, nb = p.B * (bgi + 1) / bg - blo;
      const int sz = nh * nb;
      if (task >= sz * p.nC) return;               // past the class's tasks (uniform in the workgroup)
      c = task / sz;
      const int r = task - c * sz;
      s = (blo + r / nh) * p.H + hlo + r % nh;
    } else {
      c = task / BH;
      s = task % BH;
    }
  }
  const int b = s / p.H, h = s % p.H;
  const int c0 = c * T;
  const int Tc = min(T, p.L - c0);
  const size_t gbase = (size_t)s * p.L + c0;

  const int gpw = 64 / NP;                 // lane groups per wave
  const int gl = lane / NP, j = lane % NP;
  const int gam = wave * gpw + gl;         // this lane's group (sub-chunk)
  const int tb = gam * S, te = min(tb + S, Tc);
  const int nst = max(te - tb, 0);         // steps of this group
  const bool act = NPT ? true : (j < N);
  const int jj = act ? j : 0;              // row index that is safe to look up

  // ---- step-major selection (kSelStep32: N = 32, K <= 16, per-head bf16 u,
  // d = 128, at most two tiles of 16 steps per group).  Row i of a wave's
  // 32x32 tile kt is step 16 kt + ((i >> 3) << 2 | (i & 3)) of the wave's
  // group (i >> 2) & 1, so output element r of lane (group g, row j) is step
  // 16 kt + r of group g at column j.  One tile has the pre-activation
  // columns (rows of W_d), the other the score columns (rows of W_sel,
  // repeated in both 16-lane halves): every lane receives D_t[j] for its own
  // steps and each 16-lane row all scores of its group's steps, so the
  // selections never pass through LDS.  Weights and the wave's u tiles are
  // loaded once, as MFMA operands (lane l: column or row l % 32, channels
  // 16 m + 8 (l / 32) .. +7 of k-step m).
  constexpr bool SM32 = PATH == kSelStep32;
  constexpr int kS32 = 8;                          // 16-channel k-steps (d = 128)
  [[maybe_unused]] u4v wz32[SM32 ? kS32 : 1], ws32[SM32 ? kS32 : 1], U32[SM32 ? 2 : 1][SM32 ? kS32 : 1];
  [[maybe_unused]] float bdz32 = 0.f;
  // steps of the wave's first group (the most in the wave), uniform
  [[maybe_unused]] const int wave_nst = max(min(wave * gpw * S + S, Tc) - wave * gpw * S, 0);
  [[maybe_unused]] auto issue32 = [&]() __attribute__((always_inline)) {
    if constexpr (SM32) {
      const int col = lane & 31, kh = lane >> 5, sc = col & 15;
      const rsrc_t wzr = make_rsrc((const uint16_t*)a.W_d + (size_t)h * N * 128, (uint32_t)(N * 128 * 2));
      const rsrc_t wsr = make_rsrc((const uint16_t*)a.W_sel + (size_t)h * K * 128, (uint32_t)(K * 128 * 2));
#pragma unroll
      for (int m = 0; m < kS32; ++m) {
        wz32[m] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                              wzr, (uint32_t)((col * 128 + 16 * m + 8 * kh) * 2), 0, 0));
        ws32[m] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                              wsr, sc < K ? (uint32_t)((sc * 128 + 16 * m + 8 * kh) * 2) : kNoLoad,
                                              0, 0));
      }
      bdz32 = buf_f32(make_rsrc(a.b_d + (size_t)h * N, (uint32_t)(N * 4)), (uint32_t)col * 4u);
      const rsrc_t ur = make_rsrc((const uint16_t*)a.u + gbase * 128, (uint32_t)(Tc * 128 * 2));
      const int i = lane & 31, grp = (i >> 2) & 1, st = ((i >> 3) << 2) | (i & 3);
      const int gtb = (wave * 2 + grp) * S;          // first step of that group
      const int gns = max(min(gtb + S, Tc) - gtb, 0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int m = 0; m < kS32; ++m) {
          const bool ok = 16 * kt + st < gns;
          U32[kt][m] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                   ur, ok ? (uint32_t)(((gtb + 16 * kt + st) * 128 + 16 * m + 8 * kh) * 2)
                                                          : kNoLoad, 0, 0));
        }
    }
  };
  // pre-activations and scores of one tile
  [[maybe_unused]] auto mma32 = [&](f16v& aD, f16v& aS, const u4v* Ua) __attribute__((always_inline)) {
    if constexpr (SM32) {
      aD = f16v{};
      aS = f16v{};
#pragma unroll
      for (int m = 0; m < kS32; ++m) {
        aD = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, Ua[m]), __builtin_bit_cast(bf8v, wz32[m]),
                                                     aD, 0, 0, 0);
        aS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8v, Ua[m]), __builtin_bit_cast(bf8v, ws32[m]),
                                                     aS, 0, 0, 0);
      }
    }
  };

  // ---- phase-A drive terms of the first block: issued first, used last
  // (selection mode never reads Bu, and with the drive folded it is formed
  // on chip: Bu may be null there, and the empty descriptor loads zeros)
  const bool no_bu = MODE == kModeSelect || fold;
  const rsrc_t bur = make_rsrc(no_bu ? (const float*)nullptr : a.Bu + gbase * N,
                               no_bu ? 0u : (uint32_t)(Tc * N * 4));
  // (the deep selection path needs the registers itself: its first block
  // follows the selection instead)
  float bu[kBuBlock];
  auto first_bu = [&]() {
#pragma unroll
    for (int q = 0; q < kBuBlock; ++q)
      bu[q] = buf_f32(bur, (act && q < nst) ? (uint32_t)((tb + q) * N + j) * 4u : kNoLoad);
  };
  if constexpr (MODE != kModeSelect && PATH < kSelDeep) first_bu();

  // ---- scan alone, N = 32 or 64: the chunk's k* and D are requested before
  // the tables are built (one memory round trip for all of them; written to
  // LDS after the tables), when they fit kScanPre 16-byte loads per thread
  constexpr int kScanPre = 8;
  [[maybe_unused]] const bool pre = MODE == kModeScan && (NPT == 32 || NPT == 64) && !a.P_in &&
                                    Tc <= kThreads && Tc * N <= kScanPre * 4 * kThreads;
  [[maybe_unused]] f4v dpre[MODE == kModeScan ? kScanPre : 1];
  [[maybe_unused]] int kpre = 0;
  [[maybe_unused]] float cpre = 0.f;
  if constexpr (MODE == kModeScan && (NPT == 32 || NPT == 64)) {
    if (pre) {
      const rsrc_t dd = make_rsrc(a.D_in + gbase * N, (uint32_t)(Tc * N * 4));
#pragma unroll
      for (int e = 0; e < kScanPre; ++e) {
        const int q = e * kThreads + tid;          // 16-byte piece q of the chunk's [Tc][N] rows
        dpre[e] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(
                                              dd, 4 * q < Tc * N ? (uint32_t)q * 16u : kNoLoad, 0, 0));
      }
      kpre = buf_i32(make_rsrc(a.k_in + gbase, (uint32_t)(Tc * 4)), tid < Tc ? (uint32_t)tid * 4u : kNoLoad);
    }
  }
  // C in a register from the start (scan and fused modes, P N <= 256), so
  // that building the tables does not wait on it
  [[maybe_unused]] const bool cearly = MODE != kModeSelect && P * N <= kThreads;
  if (cearly)
    cpre = buf_f32(make_rsrc(a.C + (size_t)h * P * N, (uint32_t)(P * N * 4)), tid < P * N ? (uint32_t)tid * 4u : kNoLoad);

  // ---- per-head constants
  if constexpr (MODE == kModeSelect) {
    if (a.P_out)
      for (int q = tid; q < K * N; q += kThreads) dic[q] = a.dict[(size_t)h * K * N + q];
  } else {
    if (!cearly) {
      for (int q = tid; q < P * N; q += kThreads) Cs[q] = a.C[(size_t)h * P * N + q];
      __syncthreads();
    }
    // DR[k][m] = dict[k][m]: the target row of source m under entry k; with
    // per-step maps, entry t is step t's map and k*_t = t
    if (MODE == kModeScan && a.P_in) {
      for (int q = tid; q < Tc * N; q += kThreads)
        DR[(q / N) * p.DCS + q % N] = (unsigned char)a.P_in[gbase * N + q];
    } else if ((NPT == 32 || NPT == 64) && p.gse) {
      // the target rows and the inverse rows from one read of the dictionary;
      // every load of the wave is issued before the first ballot waits
      constexpr int NG = NPT == 64 ? 64 : 32;
      constexpr int kIt = 64 * 64 / kThreads;      // K * N / kThreads at most (K <= 64)
      i2v* SE = (i2v*)(smem + p.off_SRC);
      const rsrc_t dr = make_rsrc(a.dict + (size_t)h * K * N, (uint32_t)(K * N * 4));
      int rv[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int q = wave * 64 + it * kThreads + lane;
        rv[it] = buf_i32(dr, q < K * N ? (uint32_t)q * 4u : kNoLoad);
      }
      issue32();                                   // step-major selection operands (the table build waits only for rv)
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int q0 = wave * 64 + it * kThreads;   // uniform in the wave
        if (q0 >= K * N) break;
        const int q = q0 + lane;
        const bool on = q < K * N;
        const int r = on ? rv[it] : 0;
        if (on) DR[(q / N) * p.DCS + q % N] = (unsigned char)r;
        const i2v e = row_entry<NG>(r, on, q, lane);
        if (on) SE[q] = e;
      }
    } else {
      for (int q = tid; q < K * N; q += kThreads)
        DR[(q / N) * p.DCS + q % N] = (unsigned char)a.dict[(size_t)h * K * N + q];
    }
  }
  if constexpr (MODE == kModeScan && (NPT == 32 || NPT == 64)) {
    if (pre) {
      if (tid < Tc) kbuf[tid] = kpre;
#pragma unroll
      for (int e = 0; e < kScanPre; ++e) {
        const int q = e * kThreads + tid;
        if (4 * q < Tc * N) {
          const int t = (4 * q) / NPT, n = (4 * q) % NPT;   // four consecutive n of step t
          Dbuf[(n + 0) * TS + t] = dpre[e].x;
          Dbuf[(n + 1) * TS + t] = dpre[e].y;
          Dbuf[(n + 2) * TS + t] = dpre[e].z;
          Dbuf[(n + 3) * TS + t] = dpre[e].w;
        }
      }
    }
  }
  if (MODE == kModeScan && !pre) {
    for (int q = tid; q < Tc; q += kThreads) kbuf[q] = a.P_in ? q : a.k_in[gbase + q];
    // D of the chunk, eight loads in flight per lane at a time
    const rsrc_t dd = make_rsrc(a.D_in + gbase * N, (uint32_t)(Tc * N * 4));
    for (int q0 = 0; q0 < Tc * N; q0 += 8 * kThreads) {
      float dv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * kThreads + tid;
        dv[e] = buf_f32(dd, q < Tc * N ? (uint32_t)q * 4u : kNoLoad);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * kThreads + tid;
        if (q < Tc * N) {
          const int t = q / N, n = q - t * N;
          Dbuf[n * TS + t] = dv[e];
        }
      }
    }
  }
  if (cearly && tid < P * N) Cs[tid] = cpre;
  __syncthreads();

  // ---- selection for this wave's rows (the step-major path selects tile by
  // tile inside phase A)
  if constexpr (MODE != kModeScan && !SM32) {
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
    o.wst = (MODE == kModeFused && p.wst) ? smem + p.off_D : nullptr;
    o.Bubuf = fold ? Bubuf : nullptr;
    const int wr0 = min(wave * gpw * S, Tc), wr1 = min(wr0 + gpw * S, Tc);
    select_dispatch<IN_BF16, MMA_BF16, PATH, FOLD>(a, s_u, h, c0, wr0, wr1, lane, o);
  }
  if constexpr (MODE == kModeSelect) return;
  if constexpr (PATH >= kSelDeep) first_bu();
  WAVE_SYNC();   // this wave's k* / D rows are read back by its own lane groups

  // ---- phase A: each lane group runs its sub-chunk [tb, te) from a zero
  // state.  Padding steps (past te) act as the identity map.
  float* slot = slots + gam * NP;
  float cjo[NOUT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o) cjo[o] = (act && o < P) ? Cs[o * N + j] : 0.f;
  float hl = 0.f, msc = 1.f;
  int midx = jj;
  // NPT = 32 with the inverse-row table: h' = Bu + gather of D h over the
  // sources of each row (permutes); otherwise a scatter with LDS atomics
  [[maybe_unused]] const bool gs = (NPT == 32 || NPT == 64) && MODE != kModeSelect && p.gse &&
                                   !(MODE == kModeScan && a.P_in);
  [[maybe_unused]] const i2v* SE = (const i2v*)(smem + p.off_SRC);
  [[maybe_unused]] const int lb = NPT == 32 ? (lane & 32) << 2 : 0;
  // Scatter path (any N, or no gather table): LDS atomics into a per-group row.
  auto phase_a = [&]() {
  for (int blk = 0; blk < nst; blk += kBuBlock) {
    float bn[kBuBlock];
#pragma unroll
    for (int q = 0; q < kBuBlock; ++q) {
      const int tt = blk + kBuBlock + q;
      bn[q] = buf_f32(bur, (act && tt < nst) ? (uint32_t)((tb + tt) * N + j) * 4u : kNoLoad);
    }
#pragma unroll
    for (int q4 = 0; q4 < kBuBlock; q4 += 4) {
      const int nb = nst - blk - q4;          // steps left, uniform in the group
      if (nb <= 0) break;
      const int t0 = tb + blk + q4;
      const i4v k4 = *(const i4v*)(kbuf + t0);
      const f4v d4 = act ? *(const f4v*)(Dbuf + j * TS + t0) : f4v{1.f, 1.f, 1.f, 1.f};
      // drive terms: the register ring, or (drive folded) this row of the chunk's on-chip drive
      const f4v b4 = (fold && act) ? *(const f4v*)(Bubuf + j * TS + t0) : f4v{0.f, 0.f, 0.f, 0.f};
      int own[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) own[r] = DR[(r < nb ? k4[r] : 0) * p.DCS + jj];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = r < nb;
        const int t = t0 + r;
        const int k = valid ? k4[r] : 0;
        // next factor of the running map, gathered at its current rows
        const int nrow = DR[k * p.DCS + midx];
        const float dm = Dbuf[midx * TS + t];
        const float bt = fold ? b4[r] : bu[q4 + r];
        // h' = Bu + scatter(D h); one wave, so its LDS operations stay in order
        slot[j] = valid ? bt : 0.f;
        atomicAdd(&slot[(valid && act) ? own[r] : j], (valid ? d4[r] : 1.f) * hl);
        hl = slot[j];
        // compose, and record w_t = C Phi_t over column t (all lanes of the
        // group have read column t above)
        if (valid) {
          msc *= dm;
          midx = nrow;
        }
        // (row o of w_t at D's rows + N o: one [N][TS] block per row of C)
        if (valid && act) {
#pragma unroll
          for (int o = 0; o < NOUT; ++o)
            if (o < P) Dbuf[(o * N + j) * TS + t] = Cs[o * N + midx] * msc;
        }
        // local outputs C h'
#pragma unroll
        for (int o = 0; o < NOUT; ++o) {
          if (o < P) {
            if constexpr (NPT != 0) {
              const float yl = group_sum_last<NPT>(cjo[o] * hl);
              if (valid && j == NPT - 1) yloc[o * p.YS + t] = yl;
            } else {
              const float yl = group_sum_rt(cjo[o] * hl, NP);
              if (valid && j == 0) yloc[o * p.YS + t] = yl;
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kBuBlock; ++q) bu[q] = bn[q];
  }
  };
  // Gather path, groups of NG = 32 or 64 rows (every lane a row, the
  // dictionary stride NG): step t of a group reads its map row (k*_t and the
  // composed path), gathers D_t h over each row's sources, and takes D_t and
  // C at the path's current row from the lanes that hold them (permutes), so
  // no on-chip read lands on a random row.  With NG = 64 the group is the
  // wave and k*_t a scalar.  Blocks of four steps that lie wholly inside every
  // group of the wave skip the per-step validity selects.
  [[maybe_unused]] auto phase_a_gather = [&]() {
    constexpr int NG = NPT == 64 ? 64 : 32;
    constexpr int LG = NG == 64 ? 6 : 5;
    const unsigned lb4 = (unsigned)lb * 0x01010101u;
    const int lbm = lb;                            // byte offset of the group's lane 0
    const unsigned pm = (unsigned)p.pmask;
    // The table rows of the block's four entries are read before the first
    // step (they depend on k* alone), and with one row of C the block's w_t
    // are written after its last step: each step then waits on LDS once, for
    // its gather, instead of also on its table row and on its permute of C.
    // With one row of C the four local outputs are also summed together after
    // the last step (group_sum4).
    constexpr bool kDeferW = NOUT == 1;
    auto steps = [&](auto full_tag, const i4v k4, const f4v d4, const f4v b4, int t0, int q4, int nb) {
      constexpr bool FULL = decltype(full_tag)::value;
      int kk[4];
      i2v se4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int k = (FULL || r < nb) ? k4[r] : 0;
        if constexpr (NG == 64) k = __builtin_amdgcn_readfirstlane(k);   // one group per wave
        kk[r] = k;
        se4[r] = SE[(k << LG) + j];
      }
      [[maybe_unused]] float cwv[4], msv[4], ylv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = FULL || r < nb;
        const int t = t0 + r;
        const int k = kk[r];
        const int nrow = DR[(k << LG) + midx];
        const float dm = __int_as_float(__builtin_amdgcn_ds_bpermute(lbm + (midx << 2), __float_as_int(d4[r])));
        const float bt = fold ? b4[r] : bu[q4 + r];
        const i2v se = se4[r];
        const int vj = __float_as_int(d4[r] * hl);
        float hn = gather4w((unsigned)se.x | lb4, vj, bt, pm);
        if (__builtin_amdgcn_ballot_w64(se.y & 1)) {      // rows with five to eight sources
          // (bit 25, the more-than-eight flag, is bit 1 of byte 3: the permute ignores it)
          hn = gather4w((unsigned)se.y | lb4, vj, hn, pm);
          if (__builtin_amdgcn_ballot_w64((se.y >> 25) & 1u)) {   // more than eight: scan the map row
            const bool more = (se.y >> 25) & 1u;
            const unsigned char* DRk = DR + (k << LG);
            int cnt = 0;
            for (int q = 0; q < NG; ++q) {
              const bool src = (int)DRk[q] == j;
              const float gq = __int_as_float(__builtin_amdgcn_ds_bpermute(lbm | (q << 2), vj));
              cnt += src ? 1 : 0;
              hn += (more && src && cnt > 8) ? gq : 0.f;
            }
          }
        }
        if (valid) {
          hl = hn;
          msc *= dm;
          midx = nrow;
        }
        // w_t = C Phi_t, row o of C from the lane that holds C[o][midx]
        if constexpr (kDeferW) {
          cwv[r] = __int_as_float(__builtin_amdgcn_ds_bpermute(lbm + (midx << 2), __float_as_int(cjo[0])));
          msv[r] = msc;
        } else {
#pragma unroll
          for (int o = 0; o < NOUT; ++o) {
            if (o < P) {
              const float cw = __int_as_float(__builtin_amdgcn_ds_bpermute(lbm + (midx << 2), __float_as_int(cjo[o])));
              if (valid) Dbuf[(o * N + j) * TS + t] = cw * msc;
            }
          }
        }
        if constexpr (kDeferW) {
          ylv[r] = cjo[0] * hl;
        } else {
#pragma unroll
          for (int o = 0; o < NOUT; ++o) {
            if (o < P) {
              const float yl = group_sum_last<NG>(cjo[o] * hl);
              if (valid && j == NG - 1) yloc[o * p.YS + t] = yl;
            }
          }
        }
      }
      if constexpr (kDeferW) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (FULL || r < nb) Dbuf[j * TS + t0 + r] = cwv[r] * msv[r];
        // the block's local outputs: lane j < 4 of the group writes step t0 + j
        const float yl = group_sum4<NG>(ylv, lane);
        if (j < 4 && (FULL || j < nb)) yloc[t0 + j] = yl;
      }
    };
    // one block of kBuBlock steps; the step-major path passes the block's
    // selections in registers (kr, dr), the others read them from LDS
    auto run_block = [&](int blk, const int* kr, const float* dr) __attribute__((always_inline)) {
      float bn[kBuBlock];
#pragma unroll
      for (int q = 0; q < kBuBlock; ++q) {
        const int tt = blk + kBuBlock + q;
        bn[q] = buf_f32(bur, (tt < nst) ? (uint32_t)((tb + tt) * N + j) * 4u : kNoLoad);
      }
#pragma unroll
      for (int q4 = 0; q4 < kBuBlock; q4 += 4) {
        const int nb = nst - blk - q4;             // steps left, uniform in the group
        if (!__builtin_amdgcn_ballot_w64(nb > 0)) break;
        const int t0 = tb + blk + q4;
        i4v k4;
        f4v d4;
        if constexpr (SM32) {
          k4 = i4v{kr[q4], kr[q4 + 1], kr[q4 + 2], kr[q4 + 3]};
          d4 = f4v{dr[q4], dr[q4 + 1], dr[q4 + 2], dr[q4 + 3]};
        } else {
          k4 = *(const i4v*)(kbuf + t0);
          d4 = *(const f4v*)(Dbuf + j * TS + t0);
        }
        const f4v b4 = fold ? *(const f4v*)(Bubuf + j * TS + t0) : f4v{0.f, 0.f, 0.f, 0.f};
        if (!__builtin_amdgcn_ballot_w64(nb < 4))
          steps(std::true_type{}, k4, d4, b4, t0, q4, nb);
        else
          steps(std::false_type{}, k4, d4, b4, t0, q4, nb);
      }
#pragma unroll
      for (int q = 0; q < kBuBlock; ++q) bu[q] = bn[q];
    };
    if constexpr (SM32) {
      // D_t = logistic(pre-activation) per lane, k*_t by a row argmax over the
      // score columns of each 16-lane row (both rows of a group hold the same
      // scores), for the tile's 16 steps
      auto sel32 = [&](int blk, const f16v& aD, const f16v& aS, int* ks, float* Dr) __attribute__((always_inline)) {
        const int ci = lane & 15;
        int key[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Dr[r] = logistic(aD[r] + bdz32);
          key[r] = ci < K ? order_key(aS[r]) : (int)0x80000000;
        }
#pragma unroll
        for (int r4 = 0; r4 < 16; r4 += 4) {
          const int kq[4] = {key[r4], key[r4 + 1], key[r4 + 2], key[r4 + 3]};
          int kw[4];
          row_argmax4(kq, ci, kw);
#pragma unroll
          for (int e = 0; e < 4; ++e) ks[r4 + e] = kw[e];
        }
        if (a.k_out && j == 0)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (blk + r < nst) a.k_out[gbase + tb + blk + r] = ks[r];
        if (a.D_out)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (blk + r < nst) a.D_out[(gbase + tb + blk + r) * N + j] = Dr[r];
      };
      // both tiles' products are issued first: the second runs on the matrix
      // cores while the first tile's steps run on the vector units.  One copy
      // of the block code serves both tiles (the second tile's accumulators
      // move into the first's), which keeps the hot loop within the
      // instruction cache.
      f16v aD, aS, nD, nS;
      mma32(aD, aS, U32[0]);
      const int ntile = wave_nst > 16 ? 2 : 1;     // uniform in the wave
      if (ntile == 2) mma32(nD, nS, U32[1]);
      int ks[16];
      float Dr[16];
#pragma nounroll
      for (int kt = 0; kt < ntile; ++kt) {
        sel32(16 * kt, aD, aS, ks, Dr);
        run_block(16 * kt, ks, Dr);
        aD = nD;
        aS = nS;
      }
    } else {
      for (int blk = 0; blk < nst; blk += kBuBlock) run_block(blk, nullptr, nullptr);
    }
  };
  if constexpr ((NPT == 32 || NPT == 64) && MODE != kModeSelect) {
    if (gs) phase_a_gather();
    else phase_a();
  } else {
    phase_a();
  }

  chunk_tail<false>(a, smem, c, s, Tc, gbase, NP, gam, j, act, midx, msc, hl);
}

// ---------------------------------------------------------------------------
// Inverse dictionary rows for the step-major kernels (N, K <= 16).
// SE[k][i]: the source columns j (ascending) whose one sits in row i under
// dictionary entry k, packed for the step loop:
//   x  byte m (m < 4): 4 * (m-th source), the lane offset of its value
//   z  nibbles: sources 5 to 12;  w  nibbles: sources 13 to 16, count << 24
// SW[k][i]: the weight of each of the first four slots as a float, 1 where
// row i has an m-th source and 0 past its count (so a missing source costs a
// multiply by zero instead of a branch or a conversion).
// Thread tid < 16 K builds entry (k, i) = (tid / 16, tid % 16) from its
// dictionary row drow (-1 past N).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void write_se(i4v* SE, f4v* SW, int tid, const int (&drow)[16]) {
  const int iq = tid & 15;
  unsigned bx = 0, bz = 0, bw = 0;
  int n = 0;
#pragma unroll
  for (int jq = 0; jq < 16; ++jq) {
    const bool hit = drow[jq] == iq;
    bx |= (hit && n < 4) ? (unsigned)(4 * jq) << (8 * (n & 3)) : 0u;
    bz |= (hit && n >= 4 && n < 12) ? (unsigned)jq << (4 * ((n - 4) & 7)) : 0u;
    bw |= (hit && n >= 12) ? (unsigned)jq << (4 * ((n - 12) & 3)) : 0u;
    n += hit ? 1 : 0;
  }
  SE[tid] = i4v{(int)bx, 0, (int)bz, (int)(bw | ((unsigned)n << 24))};
  SW[tid] = f4v{n > 0 ? 1.f : 0.f, n > 1 ? 1.f : 0.f, n > 2 ? 1.f : 0.f, n > 3 ? 1.f : 0.f};
}

// h'_i = hn + sum over the sources j of row i (entries se, wt) of the value
// vj of lane j of this 16-lane group, gathered in ascending j.  lb4 holds the
// group's lane-0 byte offset in each of its four bytes (a multiple of 64, and
// a slot offset is below 64, so one OR places all four addresses; the permute
// reads address bits 2 to 7 only, so each byte needs just a shift).  Rows
// with more than four sources take a loop that the whole wave enters only
// when some lane needs it.
__device__ __forceinline__ float se_gather(const i4v se, const f4v wt, int vj, unsigned lb4, float hn) {
  const unsigned ax = (unsigned)se.x | lb4;
  float gv[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    gv[m] = __int_as_float(__builtin_amdgcn_ds_bpermute((int)(ax >> (8 * m)), vj));
#pragma unroll
  for (int m = 0; m < 4; ++m) hn = __builtin_fmaf(gv[m], wt[m], hn);
  const unsigned aw = (unsigned)se.w;
  if (__builtin_amdgcn_ballot_w64(aw >= (5u << 24))) {
    const int lbase = (int)(lb4 & 0xFFu);
    const int deg = (int)(aw >> 24);
    const unsigned az = (unsigned)se.z;
    for (int m = 4; m < 16; ++m) {
      const unsigned nib = m < 12 ? az >> (4 * (m - 4)) : aw >> (4 * (m - 12));
      const float gm = __int_as_float(__builtin_amdgcn_ds_bpermute(lbase | (int)((nib & 15u) << 2), vj));
      hn += m < deg ? gm : 0.f;
      if (!__builtin_amdgcn_ballot_w64(m + 1 < deg)) break;
    }
  }
  return hn;
}


// ---------------------------------------------------------------------------
// Fused pass with step-major tiles (N <= 16, K <= 16, per-head u).
//
// A wave holds four lane groups of 16 (group = lane / 16, state row j =
// lane % 16).  MFMA tile k of a wave takes, as its 16 rows, steps 4k .. 4k+3
// of each of the wave's four sub-chunks (row i <-> group i / 4, step
// 4k + i % 4).  The 16x16 output puts rows 4g .. 4g+3 of column i in lane
// (g, i): with the pre-activation columns first, lane (g, j) receives D_t[j]
// of its own group's four steps, and a row argmax over the score columns
// gives every lane of the group its k*_t.  Selections therefore never pass
// through LDS, and the next tile's MFMAs are issued before the current
// tile's scan steps so that the two overlap.
// ---------------------------------------------------------------------------
template <int IN_BF16, int MMA_BF16, int KCH, int SPLIT, int FOLD, int NOUT>
__device__ __forceinline__ void fused16_body(const Args& a, unsigned char* smem) {
  typedef typename Frag<IN_BF16, MMA_BF16>::T FT;
  constexpr int CB = kChanBlock<MMA_BF16>;
  constexpr int PER = MMA_BF16 ? 8 : 4;
  constexpr int ES = IN_BF16 ? 2 : 4;
  constexpr int SMAX = 32;                         // steps per group
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, S = p.S, T = p.chunk, TS = p.TS, d = p.d;
  const int BH = p.B * p.H;

  float* Dbuf = (float*)(smem + p.off_D);          // holds w_t
  float* yloc = (float*)(smem + p.off_yl);
  i2v* DC = (i2v*)(smem + p.off_DC);
  int* misc = (int*)(smem + p.off_misc);
  uint32_t* hdr = (uint32_t*)a.ws;

  if (tid == 0) misc[0] = (int)atomicAdd(&hdr[kWsTicket], 1u);
  __syncthreads();
  const int task = misc[0];
  const int c = task / BH, s = task % BH;
  const int h = s % p.H;
  const int c0 = c * T;
  const int Tc = min(T, p.L - c0);
  const size_t gbase = (size_t)s * p.L + c0;

  const int gl = lane >> 4, j = lane & 15;
  const int gam = wave * 4 + gl;
  const int tb = gam * S;
  const int nst = max(min(tb + S, Tc) - tb, 0);
  const bool act = j < N;
  const int jj = act ? j : 0;

  const int i = lane & 15, g = lane >> 4;
  i4v* SE = (i4v*)(smem + p.off_SRC);
  f4v* SW = (f4v*)(smem + p.off_SRC + K * 16 * 16);

  // ---- every global load of this chunk is issued before anything waits,
  // the L2-resident ones (dictionary, weights) first: loads retire in order,
  // so the table build below then waits only for them while the u and Bu
  // streams are still in flight
  // (buffer loads: a lane with nothing to load reads zero through an
  // out-of-range offset instead of branching, so every load is in flight at
  // once)
  // dictionary inputs for the on-chip tables (K, N <= 16: one entry per lane)
  const rsrc_t dr = make_rsrc(a.dict + (size_t)h * K * N, (uint32_t)(K * N * 4));
  const bool dc_on = tid < K * N, src_on = tid < K * 16;
  const int dq = buf_i32(dr, dc_on ? (uint32_t)tid * 4u : kNoLoad);
  int drow[16];
#pragma unroll
  for (int jq = 0; jq < 16; ++jq) {
    const bool ok = src_on && jq < N;
    const int v = buf_i32(dr, ok ? (uint32_t)(((tid >> 4) * N + jq) * 4) : kNoLoad);
    drow[jq] = ok ? v : -1;
  }

  // rows of C and the logistic biases next (the table build waits for C only,
  // so every load issued after it stays in flight)
  const float bdz = buf_f32(make_rsrc(a.b_d + (size_t)h * N, (uint32_t)(N * 4)), i < N ? (uint32_t)i * 4u : kNoLoad);
  // rows of C (NOUT > 1: p.n_out of them, C[h][o][j]); row 0 also feeds DC
  const int P = NOUT > 1 ? p.n_out : 1;
  float cjo[NOUT];
  {
    const rsrc_t cr = make_rsrc(a.C + (size_t)h * P * N, (uint32_t)(P * N * 4));
#pragma unroll
    for (int o = 0; o < NOUT; ++o) cjo[o] = buf_f32(cr, (act && o < P) ? (uint32_t)(o * N + j) * 4u : kNoLoad);
  }
  const float cj = cjo[0];

  // weight fragments: tile 0 = pre-activation columns, tile 1 = score columns
  // (split into bf16 pieces once per task when the products are emulated)
  constexpr int KB = SPLIT ? KCH / 2 : 1;          // 32-channel blocks
  FT wz[KCH], wsel[KCH];
  u4v wz3[KB][3], ws3[KB][3];
  {
    const rsrc_t wzr = make_rsrc((const unsigned char*)a.W_d + (size_t)h * N * d * ES, (uint32_t)(N * d * ES));
    const rsrc_t wsr = make_rsrc((const unsigned char*)a.W_sel + (size_t)h * K * d * ES, (uint32_t)(K * d * ES));
    if constexpr (SPLIT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f4v z[2], q[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ch = 32 * kb + 8 * g + 4 * hf;
          z[hf] = load_frag_buf<0, 0>(wzr, i < N ? (uint32_t)((i * d + ch) * 4) : kNoLoad);
          q[hf] = load_frag_buf<0, 0>(wsr, i < K ? (uint32_t)((i * d + ch) * 4) : kNoLoad);
        }
        split3(z[0], z[1], wz3[kb]);
        split3(q[0], q[1], ws3[kb]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < KCH; ++m) {
        const int ch = m * CB + PER * g;
        wz[m] = load_frag_buf<IN_BF16, MMA_BF16>(wzr, (i < N && ch < d) ? (uint32_t)((i * d + ch) * ES) : kNoLoad);
        wsel[m] = load_frag_buf<IN_BF16, MMA_BF16>(wsr, (i < K && ch < d) ? (uint32_t)((i * d + ch) * ES) : kNoLoad);
      }
    }
  }
  // FOLD: the drive term is a third tile, Bu = W_b u (rows of W_b as its
  // columns).  Its fragments are built like the others and parked in LDS,
  // one 16-byte slot per lane and fragment (the same for every wave), so the
  // register budget stays at three waves per SIMD; each block reads them
  // back for its MFMAs.
  constexpr int WBF = SPLIT ? 3 * KB : KCH;        // fragments per lane
  static_assert(!FOLD || WBF * (int)sizeof(FT) <= kWbFrags * 16, "W_b fragments exceed their LDS slots");
  unsigned char* wbl = smem + p.off_WB + lane * 16;
  if constexpr (FOLD) {
    const rsrc_t wbr = make_rsrc((const unsigned char*)a.W_b + (size_t)h * N * d * ES, (uint32_t)(N * d * ES));
    if constexpr (SPLIT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f4v z[2];
        u4v w3[3];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          z[hf] = load_frag_buf<0, 0>(wbr, i < N ? (uint32_t)((i * d + 32 * kb + 8 * g + 4 * hf) * 4) : kNoLoad);
        split3(z[0], z[1], w3);
#pragma unroll
        for (int q = 0; q < 3; ++q)
          if (wave == 0) *(u4v*)(wbl + (3 * kb + q) * 1024) = w3[q];
      }
    } else {
#pragma unroll
      for (int m = 0; m < KCH; ++m) {
        const int ch = m * CB + PER * g;
        const FT w = load_frag_buf<IN_BF16, MMA_BF16>(wbr, (i < N && ch < d) ? (uint32_t)((i * d + ch) * ES) : kNoLoad);
        if (wave == 0) *(FT*)(wbl + m * 1024) = w;
      }
    }
  }

  // u rows of tile k for this lane's A operand: group i / 4 of the wave,
  // step 4k + i % 4 of that group's sub-chunk
  const rsrc_t ur = make_rsrc((const unsigned char*)a.u + gbase * d * ES, (uint32_t)(Tc * d * ES));
  const int rg_tb = (wave * 4 + (i >> 2)) * S;
  const int rg_nst = max(min(rg_tb + S, Tc) - rg_tb, 0);
  auto load_tile = [&](FT* dst, int k) {
    const int st = 4 * k + (i & 3);
    const bool ok = st < rg_nst;
    if constexpr (SPLIT) {
      // fragment m: channels 32 (m / 2) + 8 g + 4 (m % 2) .. +3
      const uint32_t rb = (uint32_t)(((rg_tb + st) * d + 8 * g) * 4);
#pragma unroll
      for (int m = 0; m < KCH; ++m)
        dst[m] = load_frag_buf<0, 0>(ur, ok ? rb + (uint32_t)((32 * (m >> 1) + 4 * (m & 1)) * 4) : kNoLoad);
    } else {
      const uint32_t rb = (uint32_t)(((rg_tb + st) * d + PER * g) * ES);
#pragma unroll
      for (int m = 0; m < KCH; ++m)
        dst[m] = load_frag_buf<IN_BF16, MMA_BF16>(ur, ok ? rb + (uint32_t)(m * CB * ES) : kNoLoad);
    }
  };
  const int wave_nst = max(min(wave * 4 * S + S, Tc) - wave * 4 * S, 0);
  const int nblk = (wave_nst + 3) >> 2;            // uniform in the wave
  FT U[2][KCH];
  // unconditional (rows past the wave's steps load zeros): a load under a
  // branch makes the wait before the table build below count only the loads
  // issued on every path, which drains these tiles too
  load_tile(U[0], 0);
  load_tile(U[1], 1);

  // drive terms: a ring of four blocks of four steps; each block's slots are
  // refilled four blocks ahead
  const rsrc_t bur = make_rsrc(a.Bu + gbase * N, (uint32_t)(Tc * N * 4));
  auto bu_off = [&](int q) {
    return (act && q < nst) ? (uint32_t)((tb + q) * N + j) * 4u : kNoLoad;
  };
  // refills take no checks: a step past the group's own (another group's, or
  // zero past the chunk) is never committed, and inactive rows are never read
  const uint32_t bu_lane = (uint32_t)(tb * N + j) * 4u;
  float bu[FOLD ? 1 : 16];
  if constexpr (!FOLD) {
#pragma unroll
    for (int q = 0; q < 16; ++q) bu[q] = buf_f32(bur, bu_off(q));
  }

  // acc[0]: pre-activations, acc[1]: scores, acc[2] (FOLD): drive terms
  auto mma_tile = [&](f4v* acc, const FT* src) {
    acc[0] = f4v{0.f, 0.f, 0.f, 0.f};
    acc[1] = f4v{0.f, 0.f, 0.f, 0.f};
    if constexpr (FOLD) acc[2] = f4v{0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u4v xp[3];
        split3(src[2 * kb], src[2 * kb + 1], xp);
        mma_split3(acc[0], xp, wz3[kb]);
        mma_split3(acc[1], xp, ws3[kb]);
        if constexpr (FOLD) {
          u4v w3[3];
#pragma unroll
          for (int q = 0; q < 3; ++q) w3[q] = *(const u4v*)(wbl + (3 * kb + q) * 1024);
          mma_split3(acc[2], xp, w3);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < KCH; ++m) {
        mma_step<IN_BF16, MMA_BF16>(acc[0], src[m], wz[m]);
        mma_step<IN_BF16, MMA_BF16>(acc[1], src[m], wsel[m]);
        if constexpr (FOLD) mma_step<IN_BF16, MMA_BF16>(acc[2], src[m], *(const FT*)(wbl + m * 1024));
      }
    }
  };
  // ---- on-chip tables; they need only the dictionary and C
  // DC[k][m] = (dict[k][m], C[dict[k][m]]): target row and its output weight
  // (C[r] sits in every lane whose row index is r, so a lane permute finds it)
  {
    const float cdq = __int_as_float(__builtin_amdgcn_ds_bpermute(dq << 2, __float_as_int(cj)));
    if (dc_on) DC[(tid / N) * p.DCS + tid % N] = i2v{dq, __float_as_int(cdq)};
  }
  // SE: the inverse dictionary rows (sources of each row)
  if (src_on) write_se(SE, SW, tid, drow);
  float* Cs = (float*)(smem + p.off_C);            // NOUT > 1: row o of C at 16 o
  if (NOUT > 1 && tid < 16) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o) Cs[o * 16 + j] = cjo[o];
  }
  __syncthreads();                                 // tables ready

  f4v A[2][FOLD ? 3 : 2];
  if (nblk > 0) {
    mma_tile(A[0], U[0]);
    if (nblk > 2) load_tile(U[0], 2);
  }

  float hl = 0.f, msc = 1.f;
  int midx = jj;
  const int lbase = (lane & ~15) << 2;             // byte offset of this group's lane 0
  const unsigned lb4 = (unsigned)lbase * 0x01010101u;
  float* wrow = Dbuf + j * TS + tb + gam;          // w_t of this lane's row, step tb
  float* yrow = yloc + tb + gam;
  // steps of the last group of this wave: every group of the wave has at
  // least that many, so a block below it needs no per-step checks
  const int nst_last = max(min(wave * 4 * S + 4 * S, Tc) - (wave * 4 + 3) * S, 0);

  auto block = [&](auto full_tag, const int k) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int cu = k & 1, nx = cu ^ 1;
    if (k + 1 < nblk) {
      mma_tile(A[nx], U[nx]);                      // next tile, overlaps the scan below
      if (k + 3 < nblk) load_tile(U[nx], k + 3);
    }
    // selections of this tile: D for this lane's row, k* for its group
    float Dr[4];
    int key[4], ks[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Dr[r] = logistic(A[cu][0][r] + bdz);
      key[r] = i < K ? order_key(A[cu][1][r]) : (int)0x80000000;
    }
    row_argmax4(key, i, ks);
    const int nb = FULL ? 4 : nst - 4 * k;         // steps left in this group
    if (a.k_out && j == 0)
      for (int r = 0; r < 4 && r < nb; ++r) a.k_out[gbase + tb + 4 * k + r] = ks[r];
    if (a.D_out && act)
      for (int r = 0; r < 4 && r < nb; ++r) a.D_out[(gbase + tb + 4 * k + r) * N + j] = Dr[r];
    float yp[NOUT][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = FULL || r < nb;
      const int ksel = valid ? ks[r] : 0;
      const i4v se = SE[ksel * 16 + j];
      const f4v wt = SW[ksel * 16 + j];
      const i2v e = DC[ksel * 16 + midx];
      const float dm = __int_as_float(
          __builtin_amdgcn_ds_bpermute(lbase + (midx << 2), __float_as_int(Dr[r])));
      // h'_i = Bu_i + sum over the sources j of row i of D_j h_j
      float hn;
      if constexpr (FOLD) hn = A[cu][2][r];
      else hn = bu[(4 * k + r) & 15];
      hn = se_gather(se, wt, __float_as_int(Dr[r] * hl), lb4, hn);
      if (valid) {
        hl = hn;
        msc *= dm;
        midx = e.x;
      }
      if (valid && act) {
        wrow[4 * k + r] = __int_as_float(e.y) * msc;
#pragma unroll
        for (int o = 1; o < NOUT; ++o)
          if (o < P) wrow[o * N * TS + 4 * k + r] = Cs[o * 16 + midx] * msc;
      }
#pragma unroll
      for (int o = 0; o < NOUT; ++o) yp[o][r] = cjo[o] * hl;
    }
    // refill this block's drive-term slots with the block four ahead
    if constexpr (!FOLD) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bu[(4 * k + r) & 15] = buf_f32(bur, bu_lane + (uint32_t)((4 * k + 16 + r) * N * 4));
    }
    // local outputs of the four steps, summed over the group off the scan's
    // critical path
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float yl = group_sum<16>(yp[o][r]);
        if ((FULL || r < nb) && j == 0 && o < P) yrow[o * p.YS + 4 * k + r] = yl;
      }
  };
  if constexpr (FOLD || NOUT > 1) {
    // the same blocks unrolled by construction, each guarded by its own
    // test: with the drive tile or several rows of C the register allocator
    // then keeps the drive fragments and the extra outputs out of memory
    // (three waves per SIMD with four rows of C instead of two)
    unrolled(std::make_integer_sequence<int, SMAX / 4>{}, [&](auto kt) __attribute__((always_inline)) {
      constexpr int k = decltype(kt)::value;
      if (k < nblk) {
        if (4 * k + 4 <= nst_last)
          block(std::true_type{}, k);
        else
          block(std::false_type{}, k);
      }
    });
  } else {
#pragma unroll
    for (int k = 0; k < SMAX / 4; ++k) {
      if (k >= nblk) break;
      if (4 * k + 4 <= nst_last)
        block(std::true_type{}, k);
      else
        block(std::false_type{}, k);
    }
  }
  __syncthreads();                                 // the tables' bytes become the scratch of the steps below
  chunk_tail<true>(a, smem, c, s, Tc, gbase, 16, gam, j, act, midx, msc, hl);
}

// ---------------------------------------------------------------------------
// Scan alone with the step-major layout (N <= 16): 16-lane groups, lane j of
// a group owns state row j, and the maps of the group's steps stream through
// registers instead of an on-chip table.  PMAP = 1: step t's map is read
// whole from P_in (row of column j's one, per step); PMAP = 0: it is
// dictionary entry k*_t (K <= 16), looked up in the (row, C[row]) table.  The
// step
//   h'_i = Bu_i + sum over the columns j with idx_t[j] = i of D_t[j] h_j
// is, with a dictionary, a gather over the inverse rows (as in the fused
// pass); with per-step maps, whose inverses are not tabulated, a scatter-add
// done with DPP row rotations (no LDS, no atomics, a fixed summation order).
// Each lane also follows its column's
// path through the maps (p <- idx_t[p], scale <- D_t[p] scale) for the chunk
// summary and the output weights w_t = C Phi_t, exactly as the fused
// step-major pass does.  Everything after phase A is chunk_tail.
// ---------------------------------------------------------------------------
template <int PMAP, int NOUT, int STATES>
__device__ __forceinline__ void step16_body(const Args& a, unsigned char* smem) {
  constexpr int SMAX = 32;                         // steps per group
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, S = p.S, T = p.chunk, TS = p.TS;
  const int BH = p.B * p.H;

  float* Dbuf = (float*)(smem + p.off_D);          // holds w_t
  float* yloc = (float*)(smem + p.off_yl);
  float* Cs = (float*)(smem + p.off_C);
  i2v* DC = (i2v*)(smem + p.off_DC);
  int* misc = (int*)(smem + p.off_misc);
  uint32_t* hdr = (uint32_t*)a.ws;

  if (tid == 0) misc[0] = (int)atomicAdd(&hdr[kWsTicket], 1u);
  __syncthreads();
  const int task = misc[0];
  const int c = task / BH, s = task % BH;
  const int h = s % p.H;
  const int c0 = c * T;
  const int Tc = min(T, p.L - c0);
  const size_t gbase = (size_t)s * p.L + c0;

  const int gl = lane >> 4, j = lane & 15;
  const int gam = wave * 4 + gl;
  const int tb = gam * S;
  const int nst = max(min(tb + S, Tc) - tb, 0);
  const bool act = j < N;
  const int jj = act ? j : 0;

  // ---- every stream of the group's first 16 steps is in flight before
  // anything waits (out-of-range offsets read zero: no branches)
  const uint32_t rows = (uint32_t)(Tc * N * 4);
  const rsrc_t mr = PMAP ? make_rsrc(a.P_in + gbase * N, rows) : make_rsrc(a.k_in + gbase, (uint32_t)(Tc * 4));
  const rsrc_t dr = make_rsrc(a.D_in + gbase * N, rows);
  const rsrc_t bur = make_rsrc(a.Bu + gbase * N, rows);
  auto row_off = [&](int q) { return (act && q < nst) ? (uint32_t)((tb + q) * N + j) * 4u : kNoLoad; };
  auto map_off = [&](int q) {
    if constexpr (PMAP) return row_off(q);
    else return q < nst ? (uint32_t)(tb + q) * 4u : kNoLoad;
  };
  // refills take no checks: a step past the group's own (another group's, or
  // zero past the chunk) is never committed, and inactive rows are never read
  const uint32_t row_lane = (uint32_t)(tb * N + j) * 4u, map_lane = PMAP ? row_lane : (uint32_t)tb * 4u;
  int mi[16];                                      // P_in entry, or k*_t
  float dv[16], bu[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mi[q] = buf_i32(mr, map_off(q));
    dv[q] = buf_f32(dr, row_off(q));
    bu[q] = buf_f32(bur, row_off(q));
  }
  // rows of C (NOUT > 1: p.n_out of them, C[h][o][j]), row o at Cs[16 o]
  const int P = NOUT > 1 ? p.n_out : 1;
  float cjo[NOUT];
  {
    const rsrc_t cr = make_rsrc(a.C + (size_t)h * P * N, (uint32_t)(P * N * 4));
#pragma unroll
    for (int o = 0; o < NOUT; ++o) cjo[o] = buf_f32(cr, (act && o < P) ? (uint32_t)(o * N + j) * 4u : kNoLoad);
  }
  if (tid < 16) {
#pragma unroll
    for (int o = 0; o < NOUT; ++o) Cs[o * 16 + j] = cjo[o];
  }
  if constexpr (!PMAP) {
    // DC[k][m] = (dict[k][m], C[dict[k][m]]) and the inverse rows SE
    // (K <= 16: one entry per thread)
    const rsrc_t dr = make_rsrc(a.dict + (size_t)h * K * N, (uint32_t)(K * N * 4));
    const bool dc_on = tid < K * N, src_on = tid < K * 16;
    const int dq = buf_i32(dr, dc_on ? (uint32_t)tid * 4u : kNoLoad);
    int drow[16];
#pragma unroll
    for (int jq = 0; jq < 16; ++jq) {
      const bool ok = src_on && jq < N;
      const int v = buf_i32(dr, ok ? (uint32_t)(((tid >> 4) * N + jq) * 4) : kNoLoad);
      drow[jq] = ok ? v : -1;
    }
    __syncthreads();                               // Cs ready
    if (dc_on) DC[(tid / N) * 16 + tid % N] = i2v{dq, __float_as_int(Cs[dq])};
    if (src_on) write_se((i4v*)(smem + p.off_SRC), (f4v*)(smem + p.off_SRC + K * 16 * 16), tid, drow);
  }
  __syncthreads();
  const i4v* SE = (const i4v*)(smem + p.off_SRC);
  const f4v* SW = (const f4v*)(smem + p.off_SRC + K * 16 * 16);

  float hl = 0.f, msc = 1.f;
  int midx = jj;
  const int lbase = (lane & ~15) << 2;             // byte offset of this group's lane 0
  const unsigned lb4 = (unsigned)lbase * 0x01010101u;
  float* wrow = Dbuf + j * TS + tb + gam;          // w_t of this lane's row, step tb
  float* yrow = yloc + tb + gam;
  const int wave_nst = max(min(wave * 4 * S + S, Tc) - wave * 4 * S, 0);
  const int nblk = (wave_nst + 3) >> 2;            // uniform in the wave
  const int nst_last = max(min(wave * 4 * S + 4 * S, Tc) - (wave * 4 + 3) * S, 0);

  auto block = [&](auto full_tag, const int k) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int nb = FULL ? 4 : nst - 4 * k;         // steps left in this group
    float yp[NOUT][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = FULL || r < nb;
      const int q = (4 * k + r) & 15;
      const float dt = dv[q];
      int nidx;
      float cw, hn;
      if constexpr (PMAP) {
        // scatter-add of D_t h onto the drive term, inside the 16-lane row
        const int it = mi[q] & 15;
        nidx = __builtin_amdgcn_ds_bpermute(lbase + (midx << 2), it);
        hn = row_gather_add(bu[q], act ? it : -1, dt * hl, j);
      } else {
        // the same as a gather over the inverse dictionary row
        const int kt = mi[q];
        const i2v e = DC[kt * 16 + midx];
        nidx = e.x;
        cw = __int_as_float(e.y);
        hn = se_gather(SE[kt * 16 + j], SW[kt * 16 + j], __float_as_int(dt * hl), lb4, bu[q]);
      }
      const float dm = __int_as_float(__builtin_amdgcn_ds_bpermute(lbase + (midx << 2), __float_as_int(dt)));
      if (valid) {
        hl = hn;
        msc *= dm;
        midx = nidx;
      }
      if constexpr (PMAP) cw = Cs[midx];
      if (valid && act) {
        wrow[4 * k + r] = cw * msc;
#pragma unroll
        for (int o = 1; o < NOUT; ++o)
          if (o < P) wrow[o * N * TS + 4 * k + r] = Cs[o * 16 + midx] * msc;
      }
#pragma unroll
      for (int o = 0; o < NOUT; ++o) yp[o][r] = cjo[o] * hl;
    }
    // refill this block's slots with the block four ahead
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t q = 4 * k + 16 + r;
      mi[(4 * k + r) & 15] = buf_i32(mr, map_lane + q * (PMAP ? N * 4 : 4));
      dv[(4 * k + r) & 15] = buf_f32(dr, row_lane + q * N * 4);
      bu[(4 * k + r) & 15] = buf_f32(bur, row_lane + q * N * 4);
    }
#pragma unroll
    for (int o = 0; o < NOUT; ++o)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float yl = group_sum<16>(yp[o][r]);
        if ((FULL || r < nb) && j == 0 && o < P) yrow[o * p.YS + 4 * k + r] = yl;
      }
  };
#pragma unroll
  for (int k = 0; k < SMAX / 4; ++k) {
    if (k >= nblk) break;
    if (4 * k + 4 <= nst_last)
      block(std::true_type{}, k);
    else
      block(std::false_type{}, k);
  }
  __syncthreads();                                 // the tables' bytes become the scratch of the steps below
  chunk_tail<true>(a, smem, c, s, Tc, gbase, 16, gam, j, act, midx, msc, hl);
  if constexpr (STATES && !PMAP && NOUT == 1) {
    {
      // The state after every step as well: each group runs its sub-chunk
      // again from its true entering state (left in the slots by the steps
      // above; the plan keeps the tables for this), writing h_t directly.
      const float* slots = (const float*)(smem + p.off_slot);
      float hj = act ? slots[gam * 16 + j] : 0.f;
      const rsrc_t hr = make_rsrc(a.H_all + gbase * N, rows);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mi[q] = buf_i32(mr, map_off(q));
        dv[q] = buf_f32(dr, row_off(q));
        bu[q] = buf_f32(bur, row_off(q));
      }
      auto rblock = [&](auto full_tag, const int k) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int nb = FULL ? 4 : nst - 4 * k;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool valid = FULL || r < nb;
          const int q = (4 * k + r) & 15, kt = mi[q];
          const float hn = se_gather(SE[kt * 16 + j], SW[kt * 16 + j], __float_as_int(dv[q] * hj), lb4, bu[q]);
          if (valid) hj = hn;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hj), hr,
                                                (valid && act) ? row_lane + (uint32_t)((4 * k + r) * N * 4) : kNoLoad,
                                                0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t q = 4 * k + 16 + r;
          mi[(4 * k + r) & 15] = buf_i32(mr, map_lane + q * 4);
          dv[(4 * k + r) & 15] = buf_f32(dr, row_lane + q * N * 4);
          bu[(4 * k + r) & 15] = buf_f32(bur, row_lane + q * N * 4);
        }
      };
#pragma unroll
      for (int k = 0; k < SMAX / 4; ++k) {
        if (k >= nblk) break;
        if (4 * k + 4 <= nst_last)
          rblock(std::true_type{}, k);
        else
          rblock(std::false_type{}, k);
      }
    }
  }
}

template <int PMAP, int NOUT = 1, int STATES = 0>
__global__ __launch_bounds__(kThreads, 3) void pdssm_step16_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  step16_body<PMAP, NOUT, STATES>(a, smem);
}

// (more than two rows of C need more registers: two waves per SIMD then)
template <int IN_BF16, int MMA_BF16, int KCH, int SPLIT, int FOLD = 0, int NOUT = 1>
__global__ __launch_bounds__(kThreads, NOUT > 2 ? 2 : 3) void pdssm_fused16_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  fused16_body<IN_BF16, MMA_BF16, KCH, SPLIT, FOLD, NOUT>(a, smem);
}

// Two entry points over one body: the register-resident fp32 selection paths
// fit three waves per SIMD; the other paths get the larger register budget
// of two waves per SIMD.
template <int MODE, int IN_BF16, int MMA_BF16, int PATH, int NPT, int NOUT = 1, int FOLD = 0>
__global__ __launch_bounds__(kThreads, 3) void pdssm_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  pdssm_body<MODE, IN_BF16, MMA_BF16, PATH, NPT, NOUT, FOLD>(a, smem);
}

template <int MODE, int IN_BF16, int MMA_BF16, int PATH, int NPT, int NOUT = 1, int FOLD = 0>
__global__ __launch_bounds__(kThreads, 2) void pdssm_kernel_wide(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  pdssm_body<MODE, IN_BF16, MMA_BF16, PATH, NPT, NOUT, FOLD>(a, smem);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static inline int sel_path(const Plan& p) {
  if (p.step32) return kSelStep32;
  const int nct = p.NC >> 4;
  if (!p.in_bf16 && p.d == 64 && nct == 2) return kSelF32D64N2;
  if (!p.in_bf16 && p.d == 16 && nct == 1) return kSelF32D16N1;
  if (p.in_bf16 && p.mma_bf16 && p.d == 128 && nct == 3) return kSelBF16D128N3;
  if (p.in_bf16 && p.mma_bf16 && p.d == 128 && nct == 5) return kSelBF16D128N5;
  if (p.in_bf16 && p.mma_bf16 && p.d % 32 == 0 && p.d >= 256) {
    // at most 8 tiles (K, N <= 64), or kFoldMaxTiles with the drive folded
    const int nt = (p.N + 15) >> 4;
    const int dt = ((p.K + 15) >> 4) + nt + (p.fold_bu ? nt : 0);
    return kSelDeep + ((dt + 1) & ~1);
  }
  return kSelAny;
}

// Group width fixed at compile time when N is a power of two (the common
// case); otherwise the runtime-width body with per-lane guards.
static inline int npt_of(const Plan& p) {
  return (p.N == p.NP && (p.N == 8 || p.N == 16 || p.N == 32 || p.N == 64)) ? p.N : 0;
}

template <int MODE, int IN_BF16, int MMA_BF16, int PATH, int NPT, bool WIDE, int NOUT = 1, int FOLD = 0>
static inline void launch_kernel(const Args& a, hipStream_t st) {
  if constexpr (WIDE)
    hipLaunchKernelGGL((pdssm_kernel_wide<MODE, IN_BF16, MMA_BF16, PATH, NPT, NOUT, FOLD>), dim3(a.p.tasks),
                       dim3(kThreads), a.p.lds_bytes, st, a);
  else
    hipLaunchKernelGGL((pdssm_kernel<MODE, IN_BF16, MMA_BF16, PATH, NPT, NOUT, FOLD>), dim3(a.p.tasks),
                       dim3(kThreads), a.p.lds_bytes, st, a);
}

}  // namespace pdscan

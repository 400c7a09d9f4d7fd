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

constexpr uint64_t kTagValid = 1ull << 32;
constexpr int kSpinLimit = 1 << 22;

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

// ---------------------------------------------------------------------------
// Score GEMM for one 16-row tile: acc[ct] holds rows row0 + 4*(lane/16) + r,
// column 16*ct + lane%16 of [scores | pre-activations].
//
// fp32 MFMA (v_mfma_f32_16x16x4_f32): lane (i = lane%16, g = lane/16) feeds
// A = u[row0+i][c] and B = W[col][c] for the channel c = m + 4g + q of step q
// of group m; bf16 MFMA (v_mfma_f32_16x16x32_bf16): 8 channels m + 8g .. +7
// per lane.  Both operands use the same channel order, so the sum is the
// full contraction.
// ---------------------------------------------------------------------------
template <int IN_BF16, int MMA_BF16>
__device__ __forceinline__ void score_tile(const Args& a, int s_u, int h, int c0, int row0,
                                           int rowlim, int lane, f4v acc[8]) {
  const Plan& p = a.p;
  const int i = lane & 15, g = lane >> 4;
  const int row = row0 + i;
  const bool rv = row < rowlim;
  const int NCT = p.NC >> 4;
  const size_t urow = ((size_t)s_u * p.L + c0 + row) * p.d;
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f4v{0.f, 0.f, 0.f, 0.f};

  const int K = p.K, N = p.N, d = p.d;
  if constexpr (!MMA_BF16) {
    for (int m = 0; m < d; m += 16) {
      const int ch = m + 4 * g;
      f4v av = {0.f, 0.f, 0.f, 0.f};
      if (rv && ch < d) {
        if constexpr (IN_BF16) {
          u2v w = *(const u2v*)((const uint16_t*)a.u + urow + ch);
          av = f4v{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
        } else {
          av = *(const f4v*)((const float*)a.u + urow + ch);
        }
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        if (ct < NCT) {
          const int col = ct * 16 + i;
          f4v bv = {0.f, 0.f, 0.f, 0.f};
          if (ch < d && col < K + N) {
            const size_t wo = (col < K) ? ((size_t)h * K + col) * d : ((size_t)h * N + col - K) * d;
            const void* wb = (col < K) ? a.W_sel : a.W_d;
            if constexpr (IN_BF16) {
              u2v w = *(const u2v*)((const uint16_t*)wb + wo + ch);
              bv = f4v{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
            } else {
              bv = *(const f4v*)((const float*)wb + wo + ch);
            }
          }
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc[ct], 0, 0, 0);
        }
      }
    }
  } else {
    for (int m = 0; m < d; m += 32) {
      const int ch = m + 8 * g;
      u4v ar = {0u, 0u, 0u, 0u};
      if (rv && ch < d) ar = *(const u4v*)((const uint16_t*)a.u + urow + ch);
      const bf8v av = __builtin_bit_cast(bf8v, ar);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        if (ct < NCT) {
          const int col = ct * 16 + i;
          u4v br = {0u, 0u, 0u, 0u};
          if (ch < d && col < K + N) {
            const size_t wo = (col < K) ? ((size_t)h * K + col) * d : ((size_t)h * N + col - K) * d;
            const void* wb = (col < K) ? a.W_sel : a.W_d;
            br = *(const u4v*)((const uint16_t*)wb + wo + ch);
          }
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf8v, br),
                                                            acc[ct], 0, 0, 0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int MODE, int IN_BF16, int MMA_BF16>
__global__ __launch_bounds__(kThreads) void pdssm_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, NP = p.NP, S = p.S, T = p.chunk;
  const int BH = p.B * p.H;

  float* Dbuf = (float*)(smem + p.off_D);
  int* kbuf = (int*)(smem + p.off_k);
  float* yloc = (float*)(smem + p.off_yl);
  int* dic = (int*)(smem + p.off_dict);
  float* Cs = (float*)(smem + p.off_C);
  float* bds = (float*)(smem + p.off_bd);
  float* slots = (float*)(smem + p.off_slot);
  int* sIdx = (int*)(smem + p.off_sIdx);
  float* sSc = (float*)(smem + p.off_sSc);
  float* sB = (float*)(smem + p.off_sB);
  int* pIdx = (int*)(smem + p.off_pIdx);
  float* pSc = (float*)(smem + p.off_pSc);
  float* pB = (float*)(smem + p.off_pB);
  float* Hs = (float*)(smem + p.off_H);
  float* tmp = (float*)(smem + p.off_tmp);
  float* stage = (float*)(smem + p.off_stage);
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

  // ---- per-head constants
  const bool need_dict = (MODE != kModeSelect) || (a.P_out != nullptr);
  if (need_dict)
    for (int q = tid; q < K * N; q += kThreads) dic[q] = a.dict[(size_t)h * K * N + q];
  for (int q = tid; q < N; q += kThreads) {
    if (MODE != kModeScan) bds[q] = a.b_d[(size_t)h * N + q];
    if (MODE != kModeSelect) Cs[q] = a.C[(size_t)h * N + q];
  }
  if constexpr (MODE == kModeScan) {
    const size_t base = (size_t)s * p.L + c0;
    for (int q = tid; q < Tc; q += kThreads) kbuf[q] = a.k_in[base + q];
    const f4v* src = (const f4v*)(a.D_in + base * N);
    if ((N & 3) == 0) {
      for (int q = tid; q < Tc * N / 4; q += kThreads) ((f4v*)Dbuf)[q] = src[q];
    } else {
      for (int q = tid; q < Tc * N; q += kThreads) Dbuf[q] = a.D_in[base * N + q];
    }
  }
  __syncthreads();

  const int gpw = 64 / NP;                       // groups per wave
  const int wrow0 = wave * gpw * S;              // this wave's rows [wrow0, wrow1)
  const int wrow1 = min(wrow0 + gpw * S, Tc);

  // ---- selection for this wave's rows
  if constexpr (MODE != kModeScan) {
    const int s_u = p.u_shared ? b : s;
    const int i = lane & 15, g = lane >> 4;
    float* st = stage + wave * 16 * p.KP;
    for (int row0 = wrow0; row0 < wrow1; row0 += 16) {
      f4v acc[8];
      score_tile<IN_BF16, MMA_BF16>(a, s_u, h, c0, row0, wrow1, lane, acc);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        if (ct < (p.NC >> 4)) {
          const int col = ct * 16 + i;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lr = 4 * g + r, row = row0 + lr;
            if (row < wrow1) {
              const float v = acc[ct][r];
              if (col < K) {
                st[lr * p.KP + col] = v;
              } else if (col < K + N) {
                const int n = col - K;
                const float dv = logistic(v + bds[n]);
                if constexpr (MODE == kModeFused) Dbuf[row * N + n] = dv;
                if (a.D_out) a.D_out[((size_t)s * p.L + c0 + row) * N + n] = dv;
              }
            }
          }
        }
      }
      WAVE_SYNC();
      int kk = 0;
      if (lane < 16 && row0 + lane < wrow1) {
        const float* sr = st + lane * p.KP;
        float best = sr[0];
        for (int k = 1; k < K; ++k) {
          const float v = sr[k];
          if (v > best) { best = v; kk = k; }        // strict: lowest index wins ties
        }
        const int row = row0 + lane;
        if constexpr (MODE == kModeFused) kbuf[row] = kk;
        if (a.k_out) a.k_out[(size_t)s * p.L + c0 + row] = kk;
      }
      if (a.P_out) {
        // lane r (< 16) holds k* of row row0 + r
        for (int r = 0; r < 16; ++r) {
          const int kr = __shfl(kk, r, 64);
          const int row = row0 + r;
          if (row < wrow1)
            for (int n = lane; n < N; n += 64)
              a.P_out[((size_t)s * p.L + c0 + row) * N + n] = dic[kr * N + n];
        }
      }
      WAVE_SYNC();
    }
  }
  if constexpr (MODE == kModeSelect) return;

  // ---- phase A: G sub-chunks of S steps, one per lane group
  const int gl = lane / NP, j = lane % NP;
  const int gam = wave * gpw + gl;
  const int tb = gam * S;
  const bool act = j < N;
  float* slot = slots + gam * NP;
  const float cj = act ? Cs[j] : 0.f;
  float hl = 0.f, msc = 1.f;
  int midx = j;
  {
    const size_t bub = ((size_t)s * p.L + c0) * N + j;
    constexpr int PF = 16;
    float cur[PF], nxt[PF];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int t = tb + q;
      cur[q] = (act && q < S && t < Tc) ? a.Bu[bub + (size_t)t * N] : 0.f;
    }
    for (int t0 = 0; t0 < S; t0 += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int tt = t0 + PF + q, t = tb + tt;
        nxt[q] = (act && tt < S && t < Tc) ? a.Bu[bub + (size_t)t * N] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int tt = t0 + q, t = tb + tt;
        const bool gv = tt < S && t < Tc;          // uniform within the group
        const bool v = act && gv;
        const int k = gv ? kbuf[t] : 0;
        const int idx = v ? dic[k * N + j] : 0;
        const float dj = v ? Dbuf[t * N + j] : 0.f;
        if (v) slot[j] = cur[q];
        WAVE_SYNC();
        if (v) atomicAdd(&slot[idx], dj * hl);
        WAVE_SYNC();
        if (v) hl = slot[j];
        float yl = v ? cj * hl : 0.f;
        for (int off = NP >> 1; off > 0; off >>= 1) yl += __shfl_xor(yl, off, NP);
        if (gv && j == 0) yloc[t] = yl;
        if (v) {
          const int nidx = dic[k * N + midx];
          msc *= Dbuf[t * N + midx];
          midx = nidx;
        }
        WAVE_SYNC();
        if (v) Dbuf[t * N + j] = Cs[midx] * msc;   // w_t = C Phi_t (row t no longer read)
      }
#pragma unroll
      for (int q = 0; q < PF; ++q) cur[q] = nxt[q];
    }
  }
  if (act) {
    sIdx[gam * N + j] = midx;
    sSc[gam * N + j] = msc;
    sB[gam * N + j] = hl;
  }
  __syncthreads();

  // ---- combine the sub-chunk summaries in order (wave 0)
  uint32_t aggI = 0;
  float aggS = 1.f, aggB = 0.f;
  if (wave == 0) {
    const bool on = lane < N;
    int ai = lane;
    float as = 1.f, ab = 0.f;
    for (int gm = 0; gm < p.G; ++gm) {
      if (on) {
        pIdx[gm * N + lane] = ai;
        pSc[gm * N + lane] = as;
        pB[gm * N + lane] = ab;
      }
      const int ni = on ? sIdx[gm * N + ai] : 0;
      const float ns = on ? sSc[gm * N + ai] * as : 0.f;
      if (on) tmp[lane] = sB[gm * N + lane];
      WAVE_SYNC();
      if (on) atomicAdd(&tmp[sIdx[gm * N + lane]], sSc[gm * N + lane] * ab);
      WAVE_SYNC();
      if (on) ab = tmp[lane];
      WAVE_SYNC();
      ai = ni;
      as = ns;
    }
    aggI = (uint32_t)ai;
    aggS = as;
    aggB = ab;

    // ---- publish this chunk's aggregate
    uint64_t* my = agg + ((size_t)c * BH + s) * 3 * N;
    if (on) {
      put_tagged(my + lane, aggI);
      put_tagged(my + N + lane, __float_as_uint(aggS));
      put_tagged(my + 2 * N + lane, __float_as_uint(aggB));
    }

    // ---- look back for the carry into this chunk
    float x = (on && a.h0) ? a.h0[(size_t)s * N + lane] : 0.f;
    int start = 0;                         // first chunk whose aggregate must be applied
    if (c > 0) {
      int q = c - 1, spins = 0;
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
          if (q == 0) { start = 0; break; }  // x already holds h0
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
    if (on) tmp[lane] = aggB;
    WAVE_SYNC();
    if (on) atomicAdd(&tmp[aggI], aggS * x);
    WAVE_SYNC();
    float xo = on ? tmp[lane] : 0.f;
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
    const float* w = Dbuf + t * N;
    const float* cr = slots + (t / S) * NP;
    float acc = yloc[t];
    for (int n = 0; n < N; ++n) acc += w[n] * cr[n];
    a.y[(size_t)s * p.L + c0 + t] = acc;
  }
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
template <int MODE>
static hipError_t launch_mode(const Args& a, hipStream_t st) {
  const Plan& p = a.p;
  dim3 grid(p.tasks), block(kThreads);
  if (MODE != kModeSelect) {
    const size_t words = p.ws_bytes / 8;
    const int cb = (int)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096);
    hipLaunchKernelGGL(clear_kernel, dim3(cb > 0 ? cb : 1), dim3(256), 0, st, (uint64_t*)a.ws, words);
  }
  if (p.in_bf16 && p.mma_bf16)
    hipLaunchKernelGGL((pdssm_kernel<MODE, 1, 1>), grid, block, p.lds_bytes, st, a);
  else if (p.in_bf16)
    hipLaunchKernelGGL((pdssm_kernel<MODE, 1, 0>), grid, block, p.lds_bytes, st, a);
  else
    hipLaunchKernelGGL((pdssm_kernel<MODE, 0, 0>), grid, block, p.lds_bytes, st, a);
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

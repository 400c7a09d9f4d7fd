// Gradient through the chunked scan for fixed selections (device code).
//
// With h_t = A_t h_{t-1} + Bu_t and y_t = C h_t, a scalar loss with
// dLoss/dy_t = g_y[t] and dLoss/dh_L = g_hL has the adjoint recurrence
//   lam_{L-1} = C g_y[L-1] + g_hL,   lam_t = C g_y[t] + A_{t+1}^T lam_{t+1},
// and dBu_t = lam_t, dD_t[j] = lam_t[idx_t[j]] h_{t-1}[j],
// dh0 = A_0^T lam_0, dC = sum over batch and steps of g_y[t] h_t.
// A_t^T of a column-one-hot-times-diagonal map is a gather,
// (A_t^T v)_j = D_t[j] v[idx_t[j]], so the adjoint runs backwards in time
// through maps (src, w, b): v -> w .* v[src] + b, which compose in O(N)
// (index gather, scale product) like the forward maps.  The three phases of
// the forward scan ("Flash PD-SSM" summary, methodology item 3) are mirrored:
// each group of a chunk composes the map of its sub-chunk from its right end,
// the groups' maps are combined right to left, the chunks' adjoint carries
// are resolved by a decoupled look-back towards later chunks, and every group
// then replays its sub-chunk from its true entering adjoint, emitting the
// gradients.  Forward states h_t are an input (the states variant of the
// forward scan writes them).
#pragma once

#include "pdscan_bwd_plan.h"
#include "pdscan_device.h"

namespace pdscan {

// value of lane `src` of this lane's group (group lanes start at `base`)
__device__ __forceinline__ float grp_gather(float v, int base, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((base + src) << 2, __float_as_int(v)));
}
__device__ __forceinline__ int grp_gather_i(int v, int base, int src) {
  return __builtin_amdgcn_ds_bpermute((base + src) << 2, v);
}

// Loads one lane keeps in flight when staging the chunk and in the replay.
constexpr int kBwdLoadBatch = 8;
// 16 nibbles mapping every row to itself.
constexpr uint64_t kIdentityNibbles = 0xFEDCBA9876543210ull;

// PK (N <= 16): dictionary rows are also kept as 64-bit words of 16 nibbles,
// which lets each lane follow its own index path in the local pass without
// cross-lane traffic (see there).
template <bool PK>
__global__ __launch_bounds__(kThreads, 2) void pdssm_bwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Plan& p = a.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, K = p.K, S = p.S, T = p.chunk, G = p.G, NP = p.NP;
  const int BH = p.B * p.H;
  int* dic = (int*)(smem + a.l.off_dic);           // [K][N] dictionary of the head
  uint64_t* dk64 = (uint64_t*)(smem + a.l.off_dk); // PK: [K] rows as nibbles
  float* Dl = (float*)(smem + a.l.off_D) + 8 * N;  // [G][GS]: group g's S rows of N diagonals
  int* kl = (int*)(smem + a.l.off_k);              // [T] selections
  float* gyl = (float*)(smem + a.l.off_gy);        // [T] output gradients
  float* Cs = (float*)(smem + a.l.off_C);
  int* sSrc = (int*)(smem + a.l.off_s);
  float* sW = (float*)(sSrc + G * N);
  float* sB = sW + G * N;
  int* pSrc = (int*)(smem + a.l.off_p);
  float* pW = (float*)(pSrc + G * N);
  float* pB = pW + G * N;
  float* slots = (float*)(smem + a.l.off_slot);    // [G][NP] entering adjoints
  float* Hs = (float*)(smem + a.l.off_H);
  float* gcs = (float*)(smem + a.l.off_gc);        // [G][N] dC partials
  int* misc = (int*)(smem + a.l.off_misc);
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* agg = (uint64_t*)(a.ws + p.ws_agg);
  uint64_t* inc = (uint64_t*)(a.ws + p.ws_inc);

  // Tickets hand out chunks from the last one down: a chunk waits only for
  // later chunks, which took their tickets first.
  if (tid == 0) misc[0] = (int)atomicAdd(&hdr[kWsTicket], 1u);
  __syncthreads();
  const int task = misc[0];
  const int c = p.nC - 1 - task / BH, s = task % BH;
  const int h = s % p.H;
  const int c0 = c * T;
  const int Tc = min(T, p.L - c0);
  const size_t gbase = (size_t)s * p.L + c0;

  // Chunk inputs to LDS.  Each pass issues one batch of loads for every
  // array (reads past a buffer's end return zero and are not stored) before
  // its first store, so a chunk of up to 2048 steps costs one memory round
  // trip.
  {
    const rsrc_t icr = make_rsrc(a.dict + (size_t)h * K * N, (uint32_t)(K * N * 4));
    const rsrc_t cr = make_rsrc(a.C + (size_t)h * N, (uint32_t)(N * 4));
    const rsrc_t kr = make_rsrc(a.k_star + gbase, (uint32_t)(Tc * 4));
    const rsrc_t gr = make_rsrc(a.g_y + gbase, (uint32_t)(Tc * 4));
    const int nD = Tc * N, SN = S * N, gpad = a.l.GS - S * N;
    const rsrc_t dr = make_rsrc(a.D + gbase * N, (uint32_t)(nD * 4));
    const bool vec = (N & 3) == 0;                 // 16-byte rows: the chunk's D is 16-byte aligned
    const int per = vec ? 4 : 1;
    constexpr int span = kThreads * kBwdLoadBatch;
    const int passes = max(max((Tc + span - 1) / span, (nD + span * per - 1) / (span * per)),
                           max((K * N + kThreads - 1) / kThreads, (N + kThreads - 1) / kThreads));
    for (int ps = 0; ps < passes; ++ps) {
      const int q1 = ps * kThreads + tid;          // dictionary and C: one entry per lane
      const int dv = buf_i32(icr, q1 < K * N ? (uint32_t)q1 * 4u : kNoLoad);
      const float cv = buf_f32(cr, q1 < N ? (uint32_t)q1 * 4u : kNoLoad);
      int kv[kBwdLoadBatch];
      float gv[kBwdLoadBatch];
      f4v v[kBwdLoadBatch];
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const int q = ps * span + u * kThreads + tid;
        kv[u] = buf_i32(kr, q < Tc ? (uint32_t)q * 4u : kNoLoad);
        gv[u] = buf_f32(gr, q < Tc ? (uint32_t)q * 4u : kNoLoad);
        const int qd = q * per;
        if (vec) {
          v[u] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(dr, qd < nD ? (uint32_t)qd * 4u : kNoLoad, 0, 0));
        } else {
          v[u] = f4v{buf_f32(dr, qd < nD ? (uint32_t)qd * 4u : kNoLoad), 0.f, 0.f, 0.f};
        }
      }
      if (q1 < K * N) dic[q1] = dv;
      if (q1 < N) Cs[q1] = cv;
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const int q = ps * span + u * kThreads + tid;
        if (q < Tc) {
          kl[q] = kv[u];
          gyl[q] = gv[u];
        }
        const int qd = q * per;
        if (qd < nD) {
          float* dst = Dl + qd + (qd / SN) * gpad;
          if (vec) *(f4v*)dst = v[u];
          else *dst = v[u].x;
        }
      }
    }
  }
  __syncthreads();
  if constexpr (PK) {
    if (tid < K) {
      uint64_t v = 0;
      for (int n = 0; n < N; ++n) v |= (uint64_t)(uint32_t)dic[tid * N + n] << (4 * n);
      dk64[tid] = v;
    }
    __syncthreads();
  }

  const int gpw = 64 / NP;
  const int gl = lane / NP, j = lane % NP;
  const int gam = wave * gpw + gl;                 // this lane's group (sub-chunk)
  const int base = lane - j;                       // first lane of the group
  const bool act = j < N;
  const int tb = gam * S, te = min(tb + S, Tc);

  // ---- local pass: the map (src, w, b) of the sub-chunk, taking the
  // adjoint entering at its right end to the one leaving on its left,
  // (M v)_j = w_j v[src_j] + b_j.
  const int nst = te - tb;
  const float cj = act ? Cs[j] : 0.f;
  const float* Dg = Dl + gam * a.l.GS - tb * N;    // Dg[t * N + i]: D_t[i] of this group
  const int jr = act ? j : 0;                      // an in-range row for idle lanes' reads
  float x = 0.f, w = act ? 1.f : 0.f;
  int src = j;
  if constexpr (PK) {
    // Lane j follows its index path forward in time: p_0 = j,
    // p_{s+1} = idx_{tb+s}[p_s].  Then src_j = p_S, w_j is the product of
    // D_{tb+s}[p_s], and b_j sums, over s, that product up to s times
    // C[p_{s+1}] g_y[tb+s] (expanding the transposed products).  Only this
    // lane's path is read: one LDS gather of D and C per step, no exchange.
    int pth = act ? j : 0;                         // idle lanes walk from row 0 with weight 0
    for (int i0 = 0; i0 < nst; i0 += kBwdLoadBatch) {
      uint64_t dk[kBwdLoadBatch];
      float gg[kBwdLoadBatch];
      int kk[kBwdLoadBatch];
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {   // unconditional reads at in-range steps
        const int t = min(tb + i0 + u, te - 1);
        kk[u] = kl[t];
        gg[u] = gyl[t];
      }
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const bool ok = i0 + u < nst;
        dk[u] = ok ? dk64[kk[u]] : kIdentityNibbles;
        gg[u] = ok ? gg[u] : 0.f;
      }
      const float* drow = Dg + (tb + i0) * N;      // rows past te-1 fall in the slack or the next group
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const float dr = drow[u * N + pth];
        w *= (i0 + u < nst) ? dr : 1.f;
        pth = (int)((dk[u] >> (4 * pth)) & 15u);
        x = __builtin_fmaf(w * Cs[pth], gg[u], x);
      }
    }
    src = pth;
  } else {
    // Generic N: the sub-chunk runs right to left, per step
    // x <- A_t^T (x + C g_y[t]) and (src, w) <- A_t^T o (src, w), through
    // gathers inside the lane group.  Operands are read a block of steps
    // ahead; steps past the left end are identity steps.
    for (int i0 = 0; i0 < nst; i0 += kBwdLoadBatch) {
      int rr[kBwdLoadBatch];
      float dd[kBwdLoadBatch], gg[kBwdLoadBatch];
      int kk[kBwdLoadBatch];
      const float* drow = Dg + (te - 1 - i0) * N + jr;   // rows before tb fall in the slack or the previous group
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {   // unconditional reads
        const int t = max(te - 1 - i0 - u, tb);
        kk[u] = kl[t];
        dd[u] = drow[-u * N];
        gg[u] = gyl[t];
      }
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const bool ok = i0 + u < nst;
        rr[u] = dic[kk[u] * N + jr];
        rr[u] = (act && ok) ? rr[u] : j;
        dd[u] = act ? (ok ? dd[u] : 1.f) : 0.f;
        gg[u] = ok ? gg[u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBwdLoadBatch; ++u) {
        const float lam = x + cj * gg[u];
        const float lr = grp_gather(lam, base, rr[u]);
        const int sr = grp_gather_i(src, base, rr[u]);
        const float wr = grp_gather(w, base, rr[u]);
        x = dd[u] * lr;
        src = sr;
        w = dd[u] * wr;
      }
    }
  }

  // ---- combine right to left: group g ends up with the map of groups
  // g..G-1 (the later groups' maps applied first); composing a o b reads b
  // at a's sources
  int cs = src;
  float cw = w, cb = x;
  for (int o = 1; o < G; o <<= 1) {
    if (act) {
      sSrc[gam * N + j] = cs;
      sW[gam * N + j] = cw;
      sB[gam * N + j] = cb;
    }
    __syncthreads();
    int ns = cs;
    float nw = cw, nb = cb;
    if (act && gam + o < G) {
      const int q = (gam + o) * N + cs;
      ns = sSrc[q];
      nw = cw * sW[q];
      nb = cw * sB[q] + cb;
    }
    __syncthreads();
    cs = ns;
    cw = nw;
    cb = nb;
  }
  if (act) {
    pSrc[gam * N + j] = cs;
    pW[gam * N + j] = cw;
    pB[gam * N + j] = cb;
  }
  __syncthreads();

  // ---- adjoint carries between chunks.  This chunk's map is published
  // first; then all lanes (NP per chunk) read the carries and maps of the
  // next later chunks in one batch.  The nearest published carry with every
  // map before it present settles the adjoint entering this chunk; without
  // one the window is read again (chunk c+1 publishes its carry without
  // waiting for this chunk, so the loop ends).
  if (wave == 0 && lane < N) {
    uint64_t* my = agg + ((size_t)c * BH + s) * 3 * N;
    put_tagged(my + lane, (uint32_t)pSrc[lane]);
    put_tagged(my + N + lane, __float_as_uint(pW[lane]));
    put_tagged(my + 2 * N + lane, __float_as_uint(pB[lane]));
  }
  const int later = p.nC - 1 - c;                  // chunks after this one
  const int wq = min(min(kThreads / NP, kBwdLookWin), later);
  int* wSrc = (int*)(smem + a.l.off_win);          // [kBwdLookWin][N] window maps and carries
  float* wW = (float*)(wSrc + kBwdLookWin * N);
  float* wB = wW + kBwdLookWin * N;
  float* wI = wB + kBwdLookWin * N;
  int* wFlag = (int*)(wI + kBwdLookWin * N);       // bit 0: carry complete, bit 1: map complete
  int hit = -1;
  for (int spins = 0; wq > 0; ++spins) {
    const int qq = tid / NP, jj = tid % NP;
    const bool in = qq < wq, on = in && jj < N;
    uint64_t iv = kTagValid, m0 = kTagValid, m1 = kTagValid, m2 = kTagValid;
    if (on) {
      const size_t cq = (size_t)(c + 1 + qq) * BH + s;
      iv = get_tagged(inc + cq * N + jj);
      m0 = get_tagged(agg + cq * 3 * N + jj);
      m1 = get_tagged(agg + cq * 3 * N + N + jj);
      m2 = get_tagged(agg + cq * 3 * N + 2 * N + jj);
      wI[qq * N + jj] = __uint_as_float((uint32_t)iv);
      wSrc[qq * N + jj] = (int)(uint32_t)m0;
      wW[qq * N + jj] = __uint_as_float((uint32_t)m1);
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
    if (hit >= 0 && !a.p.force_giveup) break;
    if (spins >= a.p.spin_limit) {                 // give up: zero carry, flag the call
      hit = -1;
      if (tid == 0) atomicOr(&hdr[kWsError], 1u);
      break;
    }
    __syncthreads();                               // the window is rewritten
    __builtin_amdgcn_s_sleep(1);
  }

  // the adjoint entering this chunk, then the one it passes on (wave 0)
  if (wave == 0) {
    const bool on = lane < N;
    const int ln = on ? lane : 0;
    float nu = (on && a.g_hL) ? a.g_hL[(size_t)s * N + lane] : 0.f;   // entering the last chunk
    if (hit >= 0) {
      // the carry of chunk c+1+hit, then the maps of chunks c+hit .. c+1
      if (on) nu = wI[hit * N + lane];
      for (int q = hit - 1; q >= 0; --q) {
        const float nv = grp_gather(nu, 0, on ? wSrc[q * N + lane] : lane);
        if (on) nu = wW[q * N + lane] * nv + wB[q * N + lane];
      }
    }
    // the adjoint this chunk passes on: its whole map applied to nu
    const float nv = grp_gather(nu, 0, on ? pSrc[ln] : lane);
    if (on) {
      put_tagged(inc + ((size_t)c * BH + s) * N + lane, __float_as_uint(pW[ln] * nv + pB[ln]));
      Hs[lane] = nu;
    }
  }
  __syncthreads();

  // ---- adjoint entering every group: the maps of the groups after it
  // applied to the chunk's entering adjoint
  if (act) {
    float v = Hs[j];
    if (gam + 1 < G) {
      const int q = (gam + 1) * N + j;
      v = pW[q] * Hs[pSrc[q]] + pB[q];
    }
    slots[gam * NP + j] = v;
  }
  __syncthreads();

  // ---- replay: every group runs its sub-chunk backwards from its true
  // entering adjoint and writes the gradients
  // The forward states of the sub-chunk, v_i = h at step te-1-i for
  // i = 0..te-tb (the last one is the state before step tb: the previous
  // chunk's last state, or h0), are read kBwdLoadBatch steps ahead of use.
  // hr covers rows gbase-1 (when the chunk has a predecessor) .. gbase+Tc-1.
  const int pre = c0 > 0 ? 1 : 0;
  const rsrc_t hr = make_rsrc(a.H_all + (gbase - pre) * N, (uint32_t)((Tc + pre) * N * 4));
  const float hinit = (act && c0 == 0 && a.h0) ? a.h0[(size_t)s * N + j] : 0.f;
  // byte offset of v_i in hr: row te-1-i+pre, kNoLoad outside
  const int h_top = ((te - 1 + pre) * N + j) * 4;
  auto h_off = [&](int i) -> uint32_t {
    return (act && i <= nst && te - 1 - i + pre >= 0) ? (uint32_t)(h_top - i * N * 4) : kNoLoad;
  };
  // gradients of the chunk through buffer stores: byte offset of (t, j) is
  // (t N + j) 4, walking down from t = te-1; idle lanes and steps past the
  // left end store to kNoLoad, which the hardware drops
  const rsrc_t bur = make_rsrc(a.g_Bu + gbase * N, (uint32_t)(Tc * N * 4));
  const rsrc_t gdr = make_rsrc(a.g_D + gbase * N, (uint32_t)(Tc * N * 4));
  const int s_top = ((te - 1) * N + j) * 4;
  float xr = act ? slots[gam * NP + j] : 0.f;
  float gc = 0.f;
  float h_cur = buf_f32(hr, h_off(0));
  float hn[kBwdLoadBatch];
#pragma unroll
  for (int u = 0; u < kBwdLoadBatch; ++u) hn[u] = buf_f32(hr, h_off(1 + u));
  for (int i0 = 0; i0 < nst; i0 += kBwdLoadBatch) {
    float hv[kBwdLoadBatch], dd[kBwdLoadBatch], gg[kBwdLoadBatch];
    int rr[kBwdLoadBatch];
    int kk[kBwdLoadBatch];
    const float* drow = Dg + (te - 1 - i0) * N + jr;
#pragma unroll
    for (int u = 0; u < kBwdLoadBatch; ++u) {   // unconditional reads
      hv[u] = hn[u];
      hn[u] = buf_f32(hr, h_off(i0 + kBwdLoadBatch + 1 + u));
      const int t = max(te - 1 - i0 - u, tb);
      kk[u] = kl[t];
      dd[u] = drow[-u * N];
      gg[u] = gyl[t];
    }
#pragma unroll
    for (int u = 0; u < kBwdLoadBatch; ++u) {
      const bool ok = i0 + u < nst;
      if constexpr (PK) rr[u] = (int)((dk64[kk[u]] >> (4 * jr)) & 15u);
      else rr[u] = dic[kk[u] * N + jr];
      rr[u] = (act && ok) ? rr[u] : j;
      dd[u] = act ? (ok ? dd[u] : 1.f) : 0.f;
      gg[u] = ok ? gg[u] : 0.f;
    }
    const int s_blk = s_top - i0 * N * 4;
#pragma unroll
    for (int u = 0; u < kBwdLoadBatch; ++u) {
      const int i = i0 + u;
      const bool ok = i < nst;
      const float lam = xr + cj * gg[u];
      const float lr = grp_gather(lam, base, rr[u]);
      const float h_prev = (c0 + te - 1 - i > 0) ? hv[u] : hinit;
      gc += gg[u] * h_cur;   // gg is zero past the left end
      const uint32_t so = (act && ok) ? (uint32_t)(s_blk - u * N * 4) : kNoLoad;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lam), bur, so, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lr * h_prev), gdr, so, 0, 0);
      h_cur = ok ? h_prev : h_cur;
      xr = dd[u] * lr;
    }
  }
  if (c == 0 && gam == 0 && act && a.g_h0) a.g_h0[(size_t)s * N + j] = xr;

  // ---- dC partial of this task, summed over the groups in a fixed order
  if (act) gcs[gam * N + j] = gc;
  __syncthreads();
  if (tid < N) {
    float acc = 0.f;
    for (int g = 0; g < G; ++g) acc += gcs[g * N + tid];
    ((float*)(a.ws + a.ws_gc))[((size_t)c * BH + s) * N + tid] = acc;
  }
}

// dC[h][n]: the tasks' partials summed over (batch, chunk) pairs.  One
// workgroup per head; for each n, P = 256 / N lanes each sum every P-th pair
// in order, then lane part 0 adds the P part sums in order (a fixed order,
// so the result does not depend on timing).
__global__ __launch_bounds__(kThreads) void pdssm_bwd_reduce_c(const float* part, float* g_C, int nC, int B,
                                                                int H, int N) {
  __shared__ float acc[kThreads];
  const int hh = blockIdx.x, tid = threadIdx.x;
  const int P = N < kThreads ? kThreads / N : 1;
  const int pairs = B * nC;
  for (int n0 = 0; n0 < N; n0 += kThreads) {
    const int n = n0 + tid % N, pp = tid / N;
    const bool on = pp < P && n < N;
    float v = 0.f;
    if (on) {
#pragma unroll 8
      for (int q = pp; q < pairs; q += P) {
        const int b = q / nC, cc = q % nC;
        v += part[((size_t)cc * B * H + (size_t)b * H + hh) * N + n];
      }
    }
    acc[tid] = v;
    __syncthreads();
    if (on && pp == 0) {
      float t = 0.f;
      for (int k = 0; k < P; ++k) t += acc[k * N + tid % N];
      g_C[(size_t)hh * N + n] = t;
    }
    __syncthreads();
  }
}

}  // namespace pdscan

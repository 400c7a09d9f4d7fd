// Sensitivity of every output to the first input, dy_t / du_0, for fixed
// selections (device code).
//
// u_0 enters only step 0, so the tangent of the state after step 0 is the
// N x d matrix J_0 = W_b + P_0 diag(D_0 (1 - D_0) h0) W_d, later steps carry it
// with the same transitions, V_t = A_t V_{t-1}, and dy_t/du_0 = C V_t.  With
// Phi_t = A_t ... A_1 this is w_t J_0 where w_t = C Phi_t, the row of output
// weights the forward scan also forms.  The three phases of the chunked scan
// ("Flash PD-SSM" summary, methodology item 3) become: per lane group, the
// weight rows of its sub-chunk by lane-local index paths; per chunk, the
// composed map and a look-back for the map entering it;
// the outputs as one K = N product per chunk, [T x N] x [N x d], on the fp32
// matrix cores.  Between chunks only PD maps travel (2N words each): the
// state entering a chunk is rebuilt as E J_0 from the composed map E, so
// nothing of the sequence is stored besides the outputs ("Breaking the
// Memory Wall" summary: exact derivatives without materialising the graph).
#pragma once

#include "pdscan_device.h"
#include "pdscan_sens_plan.h"

namespace pdscan {

// NCT = d / 16 channel tiles (1..8)
template <int NCT>
__global__ __launch_bounds__(kThreads, 2) void pdssm_sens_kernel(SensArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const SensPlan& q = a.q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = q.N, K = q.K, S = q.S, G = q.G, GS = q.GS, d = q.d, T = q.chunk;
  const int BH = q.B * q.H;
  uint64_t* dk64 = (uint64_t*)(smem + q.off_dk);   // [K] dictionary rows as nibbles
  float* Cs = (float*)(smem + q.off_C);
  int* kl = (int*)(smem + q.off_k);                // [S*G] selections of the chunk
  float* Wt = (float*)(smem + q.off_W);            // group g, step i: row g*GS + i*16: D_t, then w_t
  float* cb = (float*)(smem + q.off_cb);           // [16] step-0 coefficients D_0 (1 - D_0) h0
  int* sP = (int*)(smem + q.off_P);                // [G][16] combine scratch (rows)
  float* sS = (float*)(sP + G * kSensRow);         // [G][16] combine scratch (scales)
  int* pP = (int*)(sS + G * kSensRow);             // [G][16] inclusive prefix maps
  float* pS = (float*)(pP + G * kSensRow);
  int* gEp = (int*)(smem + q.off_V);               // [G][16] per-group maps GE and GF (phase C)
  float* gEs = (float*)(gEp + G * kSensRow);
  int* gFp = (int*)(gEs + G * kSensRow);
  float* gFs = (float*)(gFp + G * kSensRow);
  int* wIdx = (int*)(smem + q.off_win);            // [kSensWin][16] window: chunk maps
  float* wSc = (float*)(wIdx + kSensWin * kSensRow);
  int* wIi = (int*)(wSc + kSensWin * kSensRow);    // [kSensWin][16] window: inclusive maps
  float* wIs = (float*)(wIi + kSensWin * kSensRow);
  int* wFlag = (int*)(wIs + kSensWin * kSensRow);  // bit 0: inclusive map complete, bit 1: chunk map complete
  int* eP = wFlag + kSensWin;                      // [16] map entering the chunk (E)
  float* eS = (float*)(eP + kSensRow);
  int* fP = (int*)(eS + kSensRow);                 // [16] E composed with step 0's coefficient map (F)
  float* fS = (float*)(fP + kSensRow);
  int* misc = (int*)(smem + q.off_misc);
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* agg = (uint64_t*)(a.ws + q.ws_agg);
  uint64_t* inc = (uint64_t*)(a.ws + q.ws_inc);

  // tickets in chunk-major order: a chunk waits only for earlier chunks
  if (tid == 0) misc[0] = (int)atomicAdd(&hdr[kWsTicket], 1u);
  __syncthreads();
  const int task = misc[0];
  const int c = task / BH, s = task % BH;
  const int h = s % q.H;
  const int c0 = c * T;
  const int Tc = min(T, q.L - c0);
  const size_t gbase = (size_t)s * q.L + c0;

  // ---- staging: every load of the task is issued before the first wait
  // (buffer loads; a lane with nothing to load reads zero through an
  // out-of-range offset): dictionary rows, C, step 0 of the sequence (k*_0
  // and D_0, h0 for the coefficients D_0 (1 - D_0) h0 of the state tangent
  // after it), this group's k* and D rows, and phase C's operands W_b, W_d
  const int gl = lane >> 4, j = lane & 15;
  const int gam = wave * 4 + gl;
  const int tb = gam * S;
  const int nst = max(min(tb + S, Tc) - tb, 0);
  const bool act = j < N;
  float* Wg = Wt + gam * GS;
  const int i16 = lane & 15, kq = lane >> 4;
  float av[NCT][8];                                // phase C A operands: [W_b; W_d]^T
  int kv[kSensMaxS / 16];
  f4v v4[kSensMaxS * 16 / 64];                     // this group's D rows, four values per slot
  const bool vec = (N & 3) == 0;                   // 16-byte pieces never straddle a row
  const int nD = nst * N, eb = tb * N;
  {
    const rsrc_t dr = make_rsrc(a.dict + (size_t)h * K * N, (uint32_t)(K * N * 4));
    const rsrc_t cr = make_rsrc(a.C + (size_t)h * N, (uint32_t)(N * 4));
    const rsrc_t sd = make_rsrc(a.D + (size_t)s * q.L * N, (uint32_t)(N * 4));
    const rsrc_t hr = make_rsrc(a.h0 ? a.h0 + (size_t)s * N : a.C, a.h0 ? (uint32_t)(N * 4) : 0u);
    const rsrc_t kr = make_rsrc(a.k_star + gbase, (uint32_t)(Tc * 4));
    const rsrc_t k0r = make_rsrc(a.k_star + (size_t)s * q.L, 4u);
    const rsrc_t Dr = make_rsrc(a.D + gbase * N, (uint32_t)(Tc * N * 4));
    const int es = q.in_bf16 ? 2 : 4;
    const rsrc_t wbr = make_rsrc((const unsigned char*)a.W_b + (size_t)h * N * d * es, (uint32_t)(N * d * es));
    const rsrc_t wdr = make_rsrc((const unsigned char*)a.W_d + (size_t)h * N * d * es, (uint32_t)(N * d * es));
    int dn[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) dn[n] = buf_i32(dr, (tid < K && n < N) ? (uint32_t)(tid * N + n) * 4u : kNoLoad);
    const float cv = buf_f32(cr, tid < N ? (uint32_t)tid * 4u : kNoLoad);
    const float d0 = buf_f32(sd, tid < N ? (uint32_t)tid * 4u : kNoLoad);
    const float hv = buf_f32(hr, tid < N ? (uint32_t)tid * 4u : kNoLoad);
    const int k0 = buf_i32(k0r, tid == 0 ? 0u : kNoLoad);
#pragma unroll
    for (int m = 0; m < kSensMaxS / 16; ++m)
      kv[m] = buf_i32(kr, j + 16 * m < nst ? (uint32_t)(tb + j + 16 * m) * 4u : kNoLoad);
    if (vec) {
#pragma unroll
      for (int m = 0; m < kSensMaxS * 16 / 64; ++m) {
        const int e = 4 * (j + 16 * m);
        v4[m] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(Dr, e < nD ? (uint32_t)(eb + e) * 4u : kNoLoad, 0, 0));
      }
    } else {
#pragma unroll
      for (int m = 0; m < kSensMaxS * 16 / 64; ++m)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int e = j + 16 * (4 * m + q4);
          v4[m][q4] = buf_f32(Dr, e < nD ? (uint32_t)(eb + e) * 4u : kNoLoad);
        }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int kk = kb * 4 + kq, jj = kk & 15;
        const bool ok = jj < N;
        const uint32_t e = (uint32_t)(jj * d + ct * 16 + i16);
        const rsrc_t wr = kk < 16 ? wbr : wdr;
        if (q.in_bf16)
          av[ct][kb] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wr, ok ? e * 2u : kNoLoad, 0, 0) << 16);
        else
          av[ct][kb] = buf_f32(wr, ok ? e * 4u : kNoLoad);
      }
    // stores
    if (tid < K) {
      uint64_t v = 0;
#pragma unroll
      for (int n = 0; n < 16; ++n) v |= (uint64_t)(uint32_t)dn[n] << (4 * n);
      dk64[tid] = v;
    }
    if (tid < kSensRow) {
      Cs[tid] = cv;
      cb[tid] = d0 * (1.f - d0) * hv;              // zero past N (and without h0)
    }
    if (tid == 0) misc[1] = k0;
#pragma unroll
    for (int m = 0; m < kSensMaxS / 16; ++m)
      if (j + 16 * m < nst) kl[tb + j + 16 * m] = kv[m];
    if (vec) {
#pragma unroll
      for (int m = 0; m < kSensMaxS * 16 / 64; ++m) {
        const int e = 4 * (j + 16 * m);
        if (e < nD) {
          const int r = e / N;
          *(f4v*)(Wg + r * kSensRow + (e - r * N)) = v4[m];
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < kSensMaxS * 16 / 64; ++m)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int e = j + 16 * (4 * m + q4);
          if (e < nD) {
            const int r = e / N;
            Wg[r * kSensRow + (e - r * N)] = v4[m][q4];
          }
        }
    }
  }
  __syncthreads();

  // ---- phase A: lane j of group gam follows the path of row j through its
  // sub-chunk: p <- idx_t[p], scale <- D_t[p] scale, and replaces row t with
  // w_t[j] = C[p] scale (the row is read by every lane of the group before
  // any lane writes it: one wave, LDS in order).  Global step 0 is the
  // identity (the tangent starts after it).
  int pth = act ? j : 0;
  float sc = act ? 1.f : 0.f;
  for (int i0 = 0; i0 < nst; i0 += 8) {
    // per block of eight steps: the path (registers only), then every read
    // of the block, then the scales, then the block's rows are replaced
    uint64_t dk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) dk[u] = dk64[kl[tb + min(i0 + u, nst - 1)]];
    int pp[9];
    pp[0] = pth;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool adv = i0 + u < nst && c0 + tb + i0 + u > 0;
      pp[u + 1] = adv ? (int)((dk[u] >> (4 * pp[u])) & 15u) : pp[u];
    }
    float dv[8], cv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dv[u] = Wg[(i0 + u) * kSensRow + pp[u]];     // rows past nst: slack or the next group, unused
      cv[u] = Cs[pp[u + 1]];
    }
    float wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool adv = i0 + u < nst && c0 + tb + i0 + u > 0;
      sc = adv ? sc * dv[u] : sc;
      wv[u] = act ? cv[u] * sc : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u < nst) Wg[(i0 + u) * kSensRow + j] = wv[u];
    pth = pp[8];
  }

  // ---- combine: inclusive prefix of the group maps in time order (group g
  // ends with the map from the chunk start to its own end)
  int cp = pth;
  float cs = sc;
  for (int o = 1; o < G; o <<= 1) {
    sP[gam * kSensRow + j] = cp;
    sS[gam * kSensRow + j] = cs;
    __syncthreads();
    int np_ = cp;
    float ns_ = cs;
    if (act && gam >= o) {
      const int pp = sP[(gam - o) * kSensRow + j];
      const float ps = sS[(gam - o) * kSensRow + j];
      np_ = sP[gam * kSensRow + pp];
      ns_ = sS[gam * kSensRow + pp] * ps;
    }
    __syncthreads();
    cp = np_;
    cs = ns_;
  }
  pP[gam * kSensRow + j] = cp;
  pS[gam * kSensRow + j] = cs;
  __syncthreads();

  // ---- publish this chunk's map (rows and scales of the last group)
  if (wave == 0 && lane < N) {
    uint64_t* my = agg + ((size_t)c * BH + s) * 2 * N;
    put_tagged(my + lane, (uint32_t)pP[(G - 1) * kSensRow + lane]);
    put_tagged(my + N + lane, __float_as_uint(pS[(G - 1) * kSensRow + lane]));
  }

  // ---- the map entering this chunk, E = M_{c-1} o ... o M_0 (from step 1
  // to the chunk start; identity for chunk 0), composed like the forward
  // scan's carries: all lanes read the inclusive maps and chunk maps of the
  // previous chunks in one batch; the nearest complete inclusive map with
  // every chunk map after it present gives E, read again until one is
  // (chunk c-1 publishes without waiting for this chunk)
  int hit = -1;
  const int wq = min(kSensWin, c);
  for (int spins = 0; wq > 0; ++spins) {
    const int qq = tid / kSensRow, jj = tid % kSensRow;
    const bool in = qq < wq, on = in && jj < N;
    uint64_t m0 = kTagValid, m1 = kTagValid, i0 = kTagValid, i1 = kTagValid;
    if (on) {
      const size_t cq = (size_t)(c - 1 - qq) * BH + s;
      m0 = get_tagged(agg + cq * 2 * N + jj);
      m1 = get_tagged(agg + cq * 2 * N + N + jj);
      i0 = get_tagged(inc + cq * 2 * N + jj);
      i1 = get_tagged(inc + cq * 2 * N + N + jj);
      wIdx[qq * kSensRow + jj] = (int)(uint32_t)m0;
      wSc[qq * kSensRow + jj] = __uint_as_float((uint32_t)m1);
      wIi[qq * kSensRow + jj] = (int)(uint32_t)i0;
      wIs[qq * kSensRow + jj] = __uint_as_float((uint32_t)i1);
    }
    const uint64_t bi = __ballot(tag_ok(i0) && tag_ok(i1)), ba = __ballot(tag_ok(m0) && tag_ok(m1));
    if (in && jj == 0) {
      const uint64_t gm = 0xFFFFull << lane;
      wFlag[qq] = ((bi & gm) == gm ? 1 : 0) | ((ba & gm) == gm ? 2 : 0);
    }
    __syncthreads();
    for (int qx = 0; qx < wq; ++qx) {
      const int f = wFlag[qx];
      if (f & 1) { hit = qx; break; }
      if (!(f & 2)) break;
    }
    if (hit >= 0 && !a.q.force_giveup) break;
    if (spins >= a.q.spin_limit) {                 // give up: flag the call
      if (tid == 0) atomicOr(&hdr[kWsError], 1u);
      hit = 0;
      break;
    }
    __syncthreads();
    __builtin_amdgcn_s_sleep(1);
  }
  // E, the inclusive map this chunk publishes (M_c o E), and F = E o F0 with
  // F0 = (idx_0, D_0 (1 - D_0) h0), step 0's coefficient map: lane-local
  // path compositions (lanes j < N of wave 0)
  if (wave == 0 && lane < kSensRow) {
    const int jj = lane;
    int ep = jj;
    float es = jj < N ? 1.f : 0.f;
    if (hit >= 0 && jj < N) {
      ep = wIi[hit * kSensRow + jj];
      es = wIs[hit * kSensRow + jj];
      for (int qx = hit - 1; qx >= 0; --qx) {   // chunks c-hit .. c-1, oldest first
        es = wSc[qx * kSensRow + ep] * es;
        ep = wIdx[qx * kSensRow + ep];
      }
    }
    eP[jj] = ep;
    eS[jj] = es;
    const int r0 = jj < N ? (int)((dk64[misc[1]] >> (4 * jj)) & 15u) : 0;
    if (jj < N) {
      // publish M_c o E
      const int* mr = pP + (G - 1) * kSensRow;
      const float* ms = pS + (G - 1) * kSensRow;
      uint64_t* my = inc + ((size_t)c * BH + s) * 2 * N;
      put_tagged(my + jj, (uint32_t)mr[ep]);
      put_tagged(my + N + jj, __float_as_uint(ms[ep] * es));
    }
    WAVE_SYNC();
    fP[jj] = jj < N ? eP[r0] : 0;
    fS[jj] = jj < N ? eS[r0] * cb[jj] : 0.f;
  }
  __syncthreads();

  // ---- the per-group maps Phase C reads: with Pg the map from the chunk
  // start to group g's start (identity for g = 0), GE = Pg o E and
  // GF = Pg o F.  Then dy_t/du_0 = (w_t GE) W_b + (w_t GF) W_d for a step t
  // of group g, where w_t is the group-local weight row of phase A.
  {
    const int g = tid / kSensRow, jj = tid % kSensRow;
    int ep = eP[jj], fp = fP[jj];
    float es = eS[jj], fs = fS[jj];
    if (g > 0) {
      const int* gp = pP + (g - 1) * kSensRow;
      const float* gs = pS + (g - 1) * kSensRow;
      es *= gs[ep];
      ep = gp[ep];
      fs *= gs[fp];
      fp = gp[fp];
    }
    gEp[g * kSensRow + jj] = ep;
    gEs[g * kSensRow + jj] = jj < N ? es : 0.f;
    gFp[g * kSensRow + jj] = fp;
    gFs[g * kSensRow + jj] = jj < N ? fs : 0.f;
  }
  __syncthreads();

  // ---- phase C: dY[t, :] = (w_t GE) W_b + (w_t GF) W_d for the chunk's
  // steps: one 16 (channels) x 16 (steps) tile per chain of eight
  // v_mfma_f32_16x16x4_f32 over K = 32 (the rows of W_b, then of W_d); each
  // lane stores four consecutive channels of one step
  {
    const int nst16 = (Tc + 15) / 16;
    const rsrc_t yr = make_rsrc(a.dY + gbase * d, (uint32_t)(Tc * d * 4));
    for (int st = wave; st < nst16; st += kWaves) {
      const int t = min(st * 16 + i16, Tc - 1);
      const int g = t / S, ti = t - g * S;
      const float* wrow = Wt + g * GS + ti * kSensRow;
      float bw[8];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int kk = kb * 4 + kq, jj = kk & 15;
        const int mp = kk < 16 ? gEp[g * kSensRow + jj] : gFp[g * kSensRow + jj];
        const float ms = kk < 16 ? gEs[g * kSensRow + jj] : gFs[g * kSensRow + jj];
        bw[kb] = wrow[mp] * ms;                    // ms is zero for rows jj >= N
      }
      const int ts = st * 16 + i16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[ct][kb], bw[kb], acc, 0, 0, 0);
        const uint32_t off = ts < Tc ? (uint32_t)((ts * d + ct * 16 + 4 * kq) * 4) : kNoLoad;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4v, acc), yr, off, 0, 0);
      }
    }
  }
}

}  // namespace pdscan

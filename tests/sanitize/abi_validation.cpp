// The C ABI's host-side validation under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with arguments that
// must be rejected before any launch (NULL, misaligned and overlapping
// pointers, bad dims, short workspaces, unsupported shapes), and the
// workspace-size queries run on every benchmark shape and on extreme dims.
// Pointers are fake device addresses that are never dereferenced.  Exits 0
// when every case returns the expected status and no launcher was reached.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "pdscan.h"

extern int g_launches;

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, pdssm_last_error());
    ++g_fail;
  }
}

static pdssm_dims dims(int B, int H, int L, int N, int K, int d, int shared = 0, int bf = 0) {
  pdssm_dims x;
  x.B = B; x.H = H; x.L = L; x.N = N; x.K = K; x.d_in = d; x.u_shared = shared;
  x.in_dtype = bf ? PDSSM_BF16 : PDSSM_F32;
  return x;
}

static void* at(int slot) { return (void*)(uintptr_t)(0x7f0000000000ull + ((uint64_t)slot << 30)); }

int main() {
  size_t n = 0;
  // the five workload shapes and a few extreme ones: queries only
  const pdssm_dims shapes[] = {dims(1, 1, 256, 8, 4, 16), dims(4, 8, 4096, 16, 8, 64),
                               dims(8, 16, 16384, 32, 16, 128, 0, 1), dims(1, 32, 131072, 16, 8, 64),
                               dims(16, 24, 2048, 64, 32, 768, 1, 1), dims(1, 1, 1, 1, 1, 8),
                               dims(1, 1, 1 << 30, 64, 64, 8192), dims(2, 3, 1000, 17, 5, 24)};
  const int chunks[] = {1, 4, 64, 128, 256, 512, 4096};
  for (const auto& d : shapes)
    for (int c : chunks) {
      const int r1 = pdssm_fwd_workspace_bytes(&d, c, &n);
      const int r2 = pdssm_scan_workspace_bytes(&d, c, &n);
      const int r3 = pdssm_scan_bwd_workspace_bytes(&d, c, &n);
      const int r4 = pdssm_impulse_sens_workspace_bytes(&d, c, &n);
      if (r1 > 0 || r2 > 0 || r3 > 0 || r4 > 0) ++g_fail;   // statuses are <= 0
    }
  {
    const pdssm_dims d = dims(1, 32, 131072, 16, 8, 64);
    expect(pdssm_fwd_workspace_bytes(&d, 512, &n), PDSSM_OK, "impulse workspace");
    expect(n == 256 + (size_t)256 * 32 * 4 * 16 * 8 ? 0 : 1, 0, "impulse workspace size");
  }
  // bad dims and enums
  {
    int bad[][6] = {{0, 1, 1, 1, 1, 8}, {1, -1, 1, 1, 1, 8}, {1, 1, 0, 1, 1, 8},
                    {1, 1, 1, 0, 1, 8}, {1, 1, 1, 1, 0, 8}, {1, 1, 1, 1, 1, 0}};
    for (auto& b : bad) {
      const pdssm_dims d = dims(b[0], b[1], b[2], b[3], b[4], b[5]);
      expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EINVAL, "dims <= 0");
    }
    pdssm_dims d = dims(1, 1, 64, 65, 4, 16);
    expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EUNSUPPORTED, "N > 64");
    d = dims(1, 1, 64, 8, 65, 16);
    expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EUNSUPPORTED, "K > 64");
    d = dims(1, 1, 64, 8, 4, 12);
    expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EUNSUPPORTED, "d % 8");
    d = dims(1, 1, 64, 8, 4, 16);
    d.in_dtype = 7;
    expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EINVAL, "dtype");
    d = dims(1, 1, 64, 8, 4, 16);
    d.u_shared = 2;
    expect(pdssm_fwd_workspace_bytes(&d, 64, &n), PDSSM_EINVAL, "u_shared");
    d = dims(1, 1, 64, 8, 4, 16);
    expect(pdssm_fwd_workspace_bytes(&d, 0, &n), PDSSM_EINVAL, "chunk 0");
    expect(pdssm_fwd_workspace_bytes(nullptr, 16, &n), PDSSM_EINVAL, "dims NULL");
    expect(pdssm_fwd_workspace_bytes(&d, 16, nullptr), PDSSM_EINVAL, "bytes NULL");
    d = dims(1, 1, 4096, 64, 32, 64);
    expect(pdssm_fwd_workspace_bytes(&d, 4096, &n), PDSSM_EUNSUPPORTED, "on-chip footprint");
  }
  // fused entry: each required pointer NULL, misalignment, aliasing, workspace
  {
    const pdssm_dims d = dims(1, 32, 2048, 16, 8, 64);
    size_t ws = 0;
    expect(pdssm_fwd_workspace_bytes(&d, 128, &ws), PDSSM_OK, "fwd ws");
    void* p[10];
    for (int i = 0; i < 10; ++i) p[i] = at(i);
    auto call = [&](void* const* q, size_t wsb, int32_t* k = nullptr) {
      return pdssm_fwd(&d, 128, q[0], q[1], (const int32_t*)q[2], q[3], (const float*)q[4], (const float*)q[5],
                       (const float*)q[6], nullptr, k, nullptr, (float*)q[7], (float*)q[8], q[9], wsb, nullptr);
    };
    for (int i = 0; i < 10; ++i) {
      void* q[10];
      std::memcpy(q, p, sizeof q);
      q[i] = nullptr;
      expect(call(q, ws), PDSSM_EINVAL, "fwd NULL");
    }
    void* q[10];
    std::memcpy(q, p, sizeof q);
    q[5] = (char*)p[5] + 4;
    expect(call(q, ws), PDSSM_EINVAL, "fwd misaligned");
    std::memcpy(q, p, sizeof q);
    q[7] = (char*)p[5] + 64;
    expect(call(q, ws), PDSSM_EINVAL, "fwd y inside Bu");
    expect(call(p, ws, (int32_t*)p[8]), PDSSM_EINVAL, "fwd k_star on h_L");
    expect(call(p, ws - 8), PDSSM_EWORKSPACE, "fwd small workspace");
    expect(pdssm_fwd_wb(&d, 128, p[0], p[1], (const int32_t*)p[2], p[3], (const float*)p[4], nullptr,
                        (const float*)p[6], nullptr, nullptr, nullptr, (float*)p[7], (float*)p[8], p[9], ws,
                        nullptr),
           PDSSM_EINVAL, "fwd_wb W_b NULL");
  }
  // selection, scan, multi-output, states, gradient, sensitivity, soft path
  {
    const pdssm_dims d = dims(1, 32, 2048, 16, 8, 64);
    expect(pdssm_select(&d, at(0), at(1), nullptr, at(2), (const float*)at(3), (int32_t*)at(4), (float*)at(5),
                        (int32_t*)at(6), nullptr),
           PDSSM_EINVAL, "select P_idx without dict");
    expect(pdssm_select(&d, at(0), at(1), nullptr, at(2), (const float*)at(3), (int32_t*)at(4), nullptr, nullptr,
                        nullptr),
           PDSSM_EINVAL, "select D NULL");
    size_t ws = 0;
    expect(pdssm_scan_workspace_bytes(&d, 64, &ws), PDSSM_OK, "scan ws");
    expect(pdssm_scan_fwd(&d, 64, (const int32_t*)at(0), (const int32_t*)at(1), (const float*)at(2),
                          (const float*)at(3), (const float*)at(4), nullptr, (float*)at(5), (float*)at(6), at(7),
                          ws - 1, nullptr),
           PDSSM_EWORKSPACE, "scan small workspace");
    expect(pdssm_scan_fwd(&d, 64, (const int32_t*)at(0), nullptr, (const float*)at(2), (const float*)at(3),
                          (const float*)at(4), nullptr, (float*)at(5), (float*)at(6), at(7), ws, nullptr),
           PDSSM_EINVAL, "scan dict NULL");
    const int cases[][3] = {{0, 128, PDSSM_EINVAL}, {5, 128, PDSSM_EINVAL}, {2, 512, PDSSM_EUNSUPPORTED},
                            {4, 256, PDSSM_EUNSUPPORTED}, {4, 128, PDSSM_EWORKSPACE}};
    for (auto& c : cases)
      expect(pdssm_scan_fwd_multi(&d, c[1], c[0], (const int32_t*)at(0), (const int32_t*)at(1),
                                  (const float*)at(2), (const float*)at(3), (const float*)at(4), nullptr,
                                  (float*)at(5), (float*)at(6), at(7), 0, nullptr),
             c[2], "scan multi");
    expect(pdssm_scan_states(&d, 64, (const int32_t*)at(0), (const int32_t*)at(1), (const float*)at(2),
                             (const float*)at(3), (const float*)at(4), nullptr, (float*)at(5), (float*)at(6),
                             nullptr, at(7), ws, nullptr),
           PDSSM_EINVAL, "states H_all NULL");
    size_t wb = 0;
    expect(pdssm_scan_bwd_workspace_bytes(&d, 64, &wb), PDSSM_OK, "bwd ws");
    expect(pdssm_scan_bwd(&d, 64, (const int32_t*)at(0), (const int32_t*)at(1), (const float*)at(2),
                          (const float*)at(3), nullptr, (const float*)at(4), (const float*)at(5), nullptr,
                          (float*)at(6), (float*)at(7), nullptr, (float*)at(8), at(9), wb - 16, nullptr),
           PDSSM_EWORKSPACE, "bwd small workspace");
    const pdssm_dims d20 = dims(1, 2, 2048, 20, 8, 64);
    expect(pdssm_impulse_sens_workspace_bytes(&d20, 64, &wb), PDSSM_EUNSUPPORTED, "sens N > 16");
    const pdssm_dims dsh = dims(1, 2, 2048, 16, 8, 64, 1);
    expect(pdssm_impulse_sens_workspace_bytes(&dsh, 64, &wb), PDSSM_EUNSUPPORTED, "sens shared u");
    expect(pdssm_soft_select(&d, at(0), at(1), nullptr, at(2), (const float*)at(3), (float*)at(4),
                             (int32_t*)at(5), (float*)at(6), nullptr),
           PDSSM_EINVAL, "soft M NULL");
    expect(pdssm_scan_fwd_pidx(&d20, 549, (const int32_t*)at(0), (const float*)at(1), (const float*)at(2),
                               (const float*)at(3), nullptr, (float*)at(4), (float*)at(5), at(6), 1 << 20, nullptr),
           PDSSM_EUNSUPPORTED, "pidx N = 20 chunk 549");
    expect(pdssm_dict_hardmax(2, 8, 16, nullptr, (int32_t*)at(1), nullptr), PDSSM_EINVAL, "hardmax M NULL");
    expect(pdssm_workspace_status(nullptr, 4096, (uint32_t*)at(1), nullptr), PDSSM_EINVAL, "status ws NULL");
    expect(pdssm_workspace_status(at(0), 255, (uint32_t*)at(1), nullptr), PDSSM_EWORKSPACE, "status short");
  }
  std::printf("status strings: %s / %s / %s\n", pdssm_status_str(PDSSM_OK), pdssm_status_str(PDSSM_EHIP),
              pdssm_status_str(99));
  if (g_launches) {
    std::fprintf(stderr, "FAIL: %d launcher calls\n", g_launches);
    ++g_fail;
  }
  std::printf("%s: %d failures\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}

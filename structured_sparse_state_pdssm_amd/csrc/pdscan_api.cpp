// C ABI of libpdscan: argument validation (host only, before any HIP call),
// plan construction and kernel dispatch.  Declarations and the contract of
// every entry point are in include/pdscan.h.

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pdscan.h"
#include "pdscan_bwd_plan.h"
#include "pdscan_plan.h"
#include "pdscan_gemm_sel_plan.h"
#include "pdscan_sens_plan.h"
#include "pdscan_soft_plan.h"

namespace pdscan {
// One launcher per mode, each in its own translation unit.  They enqueue on
// `st` and return the launch status; scan and fused clear the workspace first.
hipError_t launch_select(const Args& a, hipStream_t st);
hipError_t launch_scan(const Args& a, hipStream_t st);
hipError_t launch_gemm_sel(const Args& a, hipStream_t st);   // pdscan_launch_gemm_sel.hip
hipError_t launch_gemm_drive(const Args& a, float* Bu, hipStream_t st);
hipError_t launch_fused(const Args& a, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, float* g_C, hipStream_t st);
hipError_t launch_sens(const SensArgs& a, hipStream_t st);
hipError_t launch_soft(const SoftArgs& a, hipStream_t st);
hipError_t launch_dict_hardmax(const float* M, int32_t* dict, int HK, int N, hipStream_t st);
hipError_t launch_status(const void* ws, uint32_t* status, hipStream_t st);
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
}

using pdscan::Plan;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

struct Range {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Shape checks common to all entry points.  `chunk` < 0 means "not used".
int check_dims(const pdssm_dims* d, int32_t chunk) {
  if (!d) return fail(PDSSM_EINVAL, "dims is NULL");
  if (d->B < 1 || d->H < 1 || d->L < 1 || d->N < 1 || d->K < 1 || d->d_in < 1)
    return fail(PDSSM_EINVAL, "dims must be >= 1 (B=%d H=%d L=%d N=%d K=%d d_in=%d)", d->B, d->H,
                d->L, d->N, d->K, d->d_in);
  if (d->u_shared != 0 && d->u_shared != 1)
    return fail(PDSSM_EINVAL, "u_shared must be 0 or 1 (got %d)", d->u_shared);
  if (d->in_dtype != PDSSM_F32 && d->in_dtype != PDSSM_BF16)
    return fail(PDSSM_EINVAL, "in_dtype must be PDSSM_F32 or PDSSM_BF16 (got %d)", d->in_dtype);
  if (chunk != -1 && chunk < 1) return fail(PDSSM_EINVAL, "chunk must be >= 1 (got %d)", chunk);
  if (d->N > 64) return fail(PDSSM_EUNSUPPORTED, "N=%d > 64 (one lane owns one state row)", d->N);
  if (d->K > 64) return fail(PDSSM_EUNSUPPORTED, "K=%d > 64", d->K);
  if (d->K + d->N > 128) return fail(PDSSM_EUNSUPPORTED, "K+N=%d > 128", d->K + d->N);
  if (d->d_in % 8 != 0) return fail(PDSSM_EUNSUPPORTED, "d_in=%d is not a multiple of 8", d->d_in);
  if (d->d_in > 8192) return fail(PDSSM_EUNSUPPORTED, "d_in=%d > 8192", d->d_in);
  const uint64_t rows = (uint64_t)d->B * d->H * d->L;
  if (rows > 0x7fffffffull)
    return fail(PDSSM_EUNSUPPORTED, "B*H*L=%llu exceeds 2^31-1", (unsigned long long)rows);
  return PDSSM_OK;
}

// Test hook: with PDSSM_TEST_LOOKBACK_GIVEUP=1 in the environment every
// look-back wait ignores the carries it finds and gives up after two window
// reads, so the workspace error word is set on purpose while every kernel
// still ends normally.  Never set in normal use.
bool lookback_giveup_hook() {
  const char* v = getenv("PDSSM_TEST_LOOKBACK_GIVEUP");
  return v && v[0] == '1' && v[1] == 0;
}

// Tuning and test hook: PDSSM_XCD_HEAD_GROUPS = 0, 1, 2, 4 or 8 overrides
// the die grouping the general fused kernel picks (0: none; a value that
// would leave a die class empty also gives none).  The results do not depend
// on it.  Returns -1 when unset.
int xcd_groups_hook() {
  const char* v = getenv("PDSSM_XCD_HEAD_GROUPS");
  if (!v || !v[0] || v[1]) return -1;
  return (v[0] == '0' || v[0] == '1' || v[0] == '2' || v[0] == '4' || v[0] == '8') ? v[0] - '0' : -1;
}

// Test hook: PDSSM_GEMM_SEL=0 keeps pdssm_select on the per-(rows, head)
// selection kernel for shapes the all-heads GEMM also takes.
int gemm_sel_hook() {
  const char* v = getenv("PDSSM_GEMM_SEL");
  return (v && v[0] == '0' && !v[1]) ? 0 : 1;
}

// Test hook: PDSSM_FWD_TWO_PASS=0 keeps pdssm_fwd on the fused kernel where
// it would otherwise run the selection GEMM and the scan as two passes.
int two_pass_hook() {
  const char* v = getenv("PDSSM_FWD_TWO_PASS");
  return (v && v[0] == '0' && !v[1]) ? 0 : 1;
}

int build_plan(Plan& p, int mode, const pdssm_dims* d, int32_t chunk, int fold_bu = 0, int step16 = 0,
               int n_out = 1) {
  const int c = (mode == pdscan::kModeSelect) ? pdscan::kSelectRows : chunk;
  if (!pdscan::make_plan(p, mode, d->B, d->H, d->L, d->N, d->K, d->d_in, d->u_shared,
                         d->in_dtype == PDSSM_BF16, c, fold_bu, step16, n_out))
    return fail(PDSSM_EUNSUPPORTED,
                "chunk=%d with N=%d needs %d bytes of on-chip memory per workgroup (limit %d)", c,
                d->N, p.lds_bytes, p.lds_limit);
  if ((uint64_t)p.nC * d->B * d->H > 0x7fffffffull)
    return fail(PDSSM_EUNSUPPORTED, "too many chunks");
  if (mode == pdscan::kModeFused && !p.fused16) {
    int hg = pdscan::xcd_head_groups(p.B, p.H, p.L, p.N, p.K, p.d, p.u_shared, p.in_bf16, p.fold_bu, p.nC);
    const int forced = xcd_groups_hook();
    if (forced >= 0) hg = (forced && forced <= p.H && pdscan::kXcds / forced <= p.B) ? forced : 0;
    if (hg && pdscan::xcd_tasks(p, hg) <= 0x7fffffffll) {
      p.xhg = hg;
      p.tasks = (int)pdscan::xcd_tasks(p, hg);
    }
  }
  if (lookback_giveup_hook()) {
    p.force_giveup = 1;
    p.spin_limit = 2;
  }
  return PDSSM_OK;
}

struct Sizes {
  size_t u, Wsel, Wd, bd, dict, Bu, C, h0, k, D, P, y, hL;
};

Sizes sizes(const pdssm_dims* d) {
  const size_t es = d->in_dtype == PDSSM_BF16 ? 2 : 4;
  const size_t B = d->B, H = d->H, L = d->L, N = d->N, K = d->K, din = d->d_in;
  Sizes s;
  s.u = B * (d->u_shared ? 1 : H) * L * din * es;
  s.Wsel = H * K * din * es;
  s.Wd = H * N * din * es;
  s.bd = H * N * 4;
  s.dict = H * K * N * 4;
  s.Bu = B * H * L * N * 4;
  s.C = H * N * 4;
  s.h0 = B * H * N * 4;
  s.k = B * H * L * 4;
  s.D = B * H * L * N * 4;
  s.P = s.D;
  s.y = B * H * L * 4;
  s.hL = B * H * N * 4;
  return s;
}

// NULL (if required), alignment and aliasing checks.
int check_ptrs(const Range* in, int nin, const Range* out, int nout, const char* const* required) {
  for (int r = 0; required[r]; ++r) {
    for (int q = 0; q < nin; ++q)
      if (!strcmp(in[q].name, required[r]) && !in[q].p)
        return fail(PDSSM_EINVAL, "%s is NULL", in[q].name);
    for (int q = 0; q < nout; ++q)
      if (!strcmp(out[q].name, required[r]) && !out[q].p)
        return fail(PDSSM_EINVAL, "%s is NULL", out[q].name);
  }
  for (int q = 0; q < nin; ++q)
    if (in[q].p && ((uintptr_t)in[q].p & 15))
      return fail(PDSSM_EINVAL, "%s is not 16-byte aligned", in[q].name);
  for (int q = 0; q < nout; ++q)
    if (out[q].p && ((uintptr_t)out[q].p & 15))
      return fail(PDSSM_EINVAL, "%s is not 16-byte aligned", out[q].name);
  for (int q = 0; q < nout; ++q) {
    for (int r = 0; r < nin; ++r)
      if (overlap(out[q], in[r]))
        return fail(PDSSM_EINVAL, "output %s overlaps input %s", out[q].name, in[r].name);
    for (int r = q + 1; r < nout; ++r)
      if (overlap(out[q], out[r]))
        return fail(PDSSM_EINVAL, "outputs %s and %s overlap", out[q].name, out[r].name);
  }
  return PDSSM_OK;
}

int dispatch(int mode, const pdscan::Args& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = mode == pdscan::kModeSelect ? pdscan::launch_select(a, st)
                       : mode == pdscan::kModeScan ? pdscan::launch_scan(a, st)
                                                   : pdscan::launch_fused(a, st);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

int sens_plan(pdscan::SensPlan& q, const pdssm_dims* dims, int32_t chunk) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  if (dims->u_shared)
    return fail(PDSSM_EUNSUPPORTED, "impulse sensitivity: u shared by the heads is not supported");
  if (dims->N > 16)
    return fail(PDSSM_EUNSUPPORTED, "impulse sensitivity: N=%d > 16", dims->N);
  if (dims->d_in % 16 || dims->d_in > pdscan::kSensMaxD)
    return fail(PDSSM_EUNSUPPORTED, "impulse sensitivity: d_in=%d must be a multiple of 16, at most %d",
                dims->d_in, pdscan::kSensMaxD);
  if (!pdscan::make_sens_plan(q, dims->B, dims->H, dims->L, dims->N, dims->K, dims->d_in,
                              dims->in_dtype == PDSSM_BF16, chunk))
    return fail(PDSSM_EUNSUPPORTED, "impulse sensitivity: chunk=%d with d_in=%d needs %d steps per lane "
                "group (at most %d: chunk <= 512) and %d bytes of on-chip memory (at most %d)", chunk,
                dims->d_in, q.S, pdscan::kSensMaxS, q.bytes, pdscan::kMaxLds);
  if ((uint64_t)q.nC * dims->B * dims->H > 0x7fffffffull)
    return fail(PDSSM_EUNSUPPORTED, "too many chunks");
  if (lookback_giveup_hook()) {
    q.force_giveup = 1;
    q.spin_limit = 2;
  }
  return PDSSM_OK;
}

}  // namespace

namespace {

// The forward passes as two passes: the all-heads selection GEMM writes k*
// and D (and, drive folded, a second GEMM writes Bu = W_b u), then the chunked
// scan reads them.  Taken for u shared by the heads with more than 32 state
// rows (the general fused kernel's deep selection there re-reads each token
// once per head and chunk task; the GEMM reads it from one die's L2 for every
// head).  Workspace: the scan's look-back words, then k*, D (used when the
// caller does not ask for them) and Bu.
bool fwd_two_pass(const pdssm_dims* d) {
  return two_pass_hook() && d->N > 32 && (long long)d->B * d->L < (1ll << 31) &&
         pdscan::gemm_sel_fits(d->u_shared, d->in_dtype == PDSSM_BF16, d->N, d->K, d->d_in);
}
struct TwoPassWs {
  size_t scan, k, D, Bu, total;   // byte offsets of k*, D and Bu, and the size
};
TwoPassWs two_pass_ws(const pdssm_dims* d, const Plan& scan) {
  TwoPassWs w;
  const size_t align = 256;
  w.scan = scan.ws_bytes;
  w.k = (w.scan + align - 1) / align * align;
  w.D = (w.k + (size_t)d->B * d->H * d->L * 4 + align - 1) / align * align;
  w.Bu = (w.D + (size_t)d->B * d->H * d->L * d->N * 4 + align - 1) / align * align;
  w.total = w.Bu + (size_t)d->B * d->H * d->L * d->N * 4;
  return w;
}

int scan_fwd_impl(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const int32_t* k_star,
                  const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                  const float* h0, float* y, float* h_L, void* workspace, size_t workspace_bytes,
                  void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeScan, dims, chunk, 0, 1, n_out))) return rc;
  if (workspace_bytes < p.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  const Sizes z = sizes(dims);
  const Range in[] = {{"k_star", k_star, z.k}, {"dict_idx", dict_idx, z.dict}, {"D", D, z.D},
                      {"Bu", Bu, z.Bu}, {"C", C, z.C * n_out}, {"h0", h0, z.h0}};
  const Range out[] = {{"y", y, z.y * n_out}, {"h_L", h_L, z.hL}, {"workspace", workspace, p.ws_bytes}};
  static const char* const req[] = {"k_star", "dict_idx", "D", "Bu", "C", "y", "h_L", "workspace",
                                    nullptr};
  if ((rc = check_ptrs(in, 6, out, 3, req))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.dict = dict_idx; a.k_in = k_star; a.D_in = D; a.Bu = Bu; a.C = C; a.h0 = h0;
  a.y = y; a.hL = h_L; a.ws = (unsigned char*)workspace;
  return dispatch(pdscan::kModeScan, a, stream);
}

int fwd_wb_impl(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const void* u, const void* W_sel,
                const int32_t* dict_idx, const void* W_d, const float* b_d, const void* W_b,
                const float* C, const float* h0, int32_t* k_star, float* D, float* y, float* h_L,
                void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  const Sizes z = sizes(dims);
  static const char* const req[] = {"u",  "W_sel", "dict_idx", "W_d", "b_d",      "W_b",
                                    "C",  "y",     "h_L",      "workspace", nullptr};
  const Range in[] = {{"u", u, z.u},         {"W_sel", W_sel, z.Wsel}, {"dict_idx", dict_idx, z.dict},
                      {"W_d", W_d, z.Wd},    {"b_d", b_d, z.bd},       {"W_b", W_b, z.Wd},
                      {"C", C, z.C * n_out}, {"h0", h0, z.h0}};
  Plan q;
  if (fwd_two_pass(dims) && build_plan(q, pdscan::kModeScan, dims, chunk, 0, 1, n_out) == PDSSM_OK) {
    // selection GEMM, drive GEMM, then the scan (with n_out rows of C)
    const TwoPassWs w = two_pass_ws(dims, q);
    if (workspace_bytes < w.total)
      return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, w.total);
    const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"y", y, z.y * n_out},
                         {"h_L", h_L, z.hL},      {"workspace", workspace, w.total}};
    if ((rc = check_ptrs(in, 8, out, 5, req))) return rc;
    unsigned char* ws = (unsigned char*)workspace;
    pdscan::Args a = {};
    a.p = q;
    a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx; a.W_b = W_b;
    a.k_out = k_star ? k_star : (int32_t*)(ws + w.k);
    a.D_out = D ? D : (float*)(ws + w.D);
    hipError_t e = pdscan::launch_gemm_sel(a, (hipStream_t)stream);
    if (e == hipSuccess) e = pdscan::launch_gemm_drive(a, (float*)(ws + w.Bu), (hipStream_t)stream);
    if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    pdscan::Args b = {};
    b.p = q;
    b.dict = dict_idx; b.k_in = a.k_out; b.D_in = a.D_out; b.Bu = (const float*)(ws + w.Bu); b.C = C;
    b.h0 = h0; b.y = y; b.hL = h_L; b.ws = ws;
    return dispatch(pdscan::kModeScan, b, stream);
  }
  g_err[0] = 0;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeFused, dims, chunk, 1, 0, n_out))) return rc;
  if (!p.fold_bu)
    return fail(PDSSM_EUNSUPPORTED,
                "the drive term cannot be folded for this shape: the selection GEMM would need more "
                "column tiles than the kernel holds (K + 2N <= 128, or with bf16 d >= 256 at most %d "
                "tiles of 16; got N=%d K=%d d=%d %s)", pdscan::kFoldMaxTiles, dims->N, dims->K,
                dims->d_in, dims->in_dtype == PDSSM_BF16 ? "bf16" : "fp32");
  if (workspace_bytes < p.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"y", y, z.y * n_out},
                       {"h_L", h_L, z.hL},      {"workspace", workspace, p.ws_bytes}};
  if ((rc = check_ptrs(in, 8, out, 5, req))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx; a.W_b = W_b;
  a.C = C; a.h0 = h0; a.k_out = k_star; a.D_out = D;
  a.y = y; a.hL = h_L; a.ws = (unsigned char*)workspace;
  return dispatch(pdscan::kModeFused, a, stream);
}

int check_n_out(int32_t n_out) {
  if (n_out < 1 || n_out > pdscan::kMaxOut)
    return fail(PDSSM_EINVAL, "n_out=%d outside [1, %d]", n_out, pdscan::kMaxOut);
  return PDSSM_OK;
}

}  // namespace

extern "C" {

int pdssm_abi_version(void) { return PDSSM_ABI_VERSION; }

int pdssm_workspace_status(const void* workspace, size_t workspace_bytes, uint32_t* status, void* stream) {
  if (!workspace) return fail(PDSSM_EINVAL, "workspace is NULL");
  if (!status) return fail(PDSSM_EINVAL, "status is NULL");
  if ((uintptr_t)workspace & 15) return fail(PDSSM_EINVAL, "workspace is not 16-byte aligned");
  if ((uintptr_t)status & 3) return fail(PDSSM_EINVAL, "status is not 4-byte aligned");
  if (workspace_bytes < 256)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes is smaller than its 256-byte header", workspace_bytes);
  const hipError_t e = pdscan::launch_status(workspace, status, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

const char* pdssm_last_error(void) { return g_err; }

const char* pdssm_status_str(int status) {
  switch (status) {
    case PDSSM_OK: return "ok";
    case PDSSM_EINVAL: return "invalid argument";
    case PDSSM_EUNSUPPORTED: return "unsupported shape";
    case PDSSM_EWORKSPACE: return "workspace too small";
    case PDSSM_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

int pdssm_select(const pdssm_dims* dims, const void* u, const void* W_sel,
                 const int32_t* dict_idx, const void* W_d, const float* b_d, int32_t* k_star,
                 float* D, int32_t* P_idx, void* stream) {
  int rc = check_dims(dims, -1);
  if (rc) return rc;
  if (P_idx && !dict_idx) return fail(PDSSM_EINVAL, "P_idx requested but dict_idx is NULL");
  const Sizes z = sizes(dims);
  const Range in[] = {{"u", u, z.u}, {"W_sel", W_sel, z.Wsel}, {"W_d", W_d, z.Wd},
                      {"b_d", b_d, z.bd}, {"dict_idx", dict_idx, z.dict}};
  const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"P_idx", P_idx, z.P}};
  static const char* const req[] = {"u", "W_sel", "W_d", "b_d", "k_star", "D", nullptr};
  if ((rc = check_ptrs(in, 5, out, 3, req))) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeSelect, dims, -1))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx;
  a.k_out = k_star; a.D_out = D; a.P_out = P_idx;
  if (gemm_sel_hook() != 0 && (long long)dims->B * dims->L < (1ll << 31) &&
      pdscan::gemm_sel_fits(dims->u_shared, dims->in_dtype == PDSSM_BF16, dims->N, dims->K, dims->d_in)) {
    // u shared by the heads: one GEMM over all tokens, the heads of a token
    // tile on one die
    const hipError_t e = pdscan::launch_gemm_sel(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PDSSM_OK;
  }
  return dispatch(pdscan::kModeSelect, a, stream);
}

int pdssm_scan_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  if (!bytes) return fail(PDSSM_EINVAL, "bytes is NULL");
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeScan, dims, chunk))) return rc;
  *bytes = p.ws_bytes;
  return PDSSM_OK;
}

int pdssm_fwd_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  if (!bytes) return fail(PDSSM_EINVAL, "bytes is NULL");
  // The size depends only on the chunk count; the shape is accepted when
  // any of the fused calls that take this workspace (pdssm_fwd, pdssm_fwd_wb,
  // pdssm_fwd_wb_multi) can run it, whose on-chip budgets differ.
  Plan p;
  rc = build_plan(p, pdscan::kModeFused, dims, chunk);
  for (int n_out = 1; rc == PDSSM_EUNSUPPORTED && n_out <= pdscan::kMaxOut; ++n_out) {
    Plan q;
    if (build_plan(q, pdscan::kModeFused, dims, chunk, 1, 0, n_out) == PDSSM_OK && q.fold_bu) {
      p = q;
      rc = PDSSM_OK;
      g_err[0] = 0;
    }
  }
  if (rc) return rc;
  *bytes = p.ws_bytes;
  if (fwd_two_pass(dims)) {
    Plan q;
    if (build_plan(q, pdscan::kModeScan, dims, chunk, 0, 1) == PDSSM_OK) {
      const size_t t = two_pass_ws(dims, q).total;
      if (t > *bytes) *bytes = t;
    }
    g_err[0] = 0;
  }
  return PDSSM_OK;
}


int pdssm_scan_fwd(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                   const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                   const float* h0, float* y, float* h_L, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return scan_fwd_impl(dims, chunk, 1, k_star, dict_idx, D, Bu, C, h0, y, h_L, workspace, workspace_bytes,
                       stream);
}

int pdssm_scan_fwd_multi(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const int32_t* k_star,
                         const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                         const float* h0, float* y, float* h_L, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int rc = check_n_out(n_out);
  if (rc) return rc;
  return scan_fwd_impl(dims, chunk, n_out, k_star, dict_idx, D, Bu, C, h0, y, h_L, workspace,
                       workspace_bytes, stream);
}

int pdssm_fwd(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
              const int32_t* dict_idx, const void* W_d, const float* b_d, const float* Bu,
              const float* C, const float* h0, int32_t* k_star, float* D, float* y, float* h_L,
              void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeFused, dims, chunk))) return rc;
  const Sizes z = sizes(dims);
  const Range in[] = {{"u", u, z.u},         {"W_sel", W_sel, z.Wsel}, {"dict_idx", dict_idx, z.dict},
                      {"W_d", W_d, z.Wd},    {"b_d", b_d, z.bd},       {"Bu", Bu, z.Bu},
                      {"C", C, z.C},         {"h0", h0, z.h0}};
  static const char* const req[] = {"u",  "W_sel", "dict_idx", "W_d", "b_d",      "Bu",
                                    "C",  "y",     "h_L",      "workspace", nullptr};
  Plan q;
  if (fwd_two_pass(dims) && build_plan(q, pdscan::kModeScan, dims, chunk, 0, 1) == PDSSM_OK) {
    const TwoPassWs w = two_pass_ws(dims, q);
    if (workspace_bytes < w.total)
      return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, w.total);
    const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"y", y, z.y},
                         {"h_L", h_L, z.hL},      {"workspace", workspace, w.total}};
    if ((rc = check_ptrs(in, 8, out, 5, req))) return rc;
    unsigned char* ws = (unsigned char*)workspace;
    pdscan::Args a = {};
    a.p = q;
    a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx;
    a.k_out = k_star ? k_star : (int32_t*)(ws + w.k);
    a.D_out = D ? D : (float*)(ws + w.D);
    hipError_t e = pdscan::launch_gemm_sel(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    pdscan::Args b = {};
    b.p = q;
    b.dict = dict_idx; b.k_in = a.k_out; b.D_in = a.D_out; b.Bu = Bu; b.C = C; b.h0 = h0;
    b.y = y; b.hL = h_L; b.ws = ws;
    return dispatch(pdscan::kModeScan, b, stream);
  }
  g_err[0] = 0;
  if (workspace_bytes < p.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"y", y, z.y},
                       {"h_L", h_L, z.hL},      {"workspace", workspace, p.ws_bytes}};
  if ((rc = check_ptrs(in, 8, out, 5, req))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx;
  a.Bu = Bu; a.C = C; a.h0 = h0; a.k_out = k_star; a.D_out = D;
  a.y = y; a.hL = h_L; a.ws = (unsigned char*)workspace;
  return dispatch(pdscan::kModeFused, a, stream);
}

int pdssm_fwd_noalloc(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
                      const int32_t* dict_idx, const void* W_d, const float* b_d, const float* Bu,
                      const float* C, const float* h0, int32_t* k_star, float* D, float* y, float* h_L,
                      uint32_t* status, void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeFused, dims, chunk))) return rc;
  if (p.ws_bytes > (size_t)PDSSM_NOALLOC_SCRATCH_BYTES)
    return fail(PDSSM_EUNSUPPORTED, "this call needs %zu bytes of look-back scratch, more than the %zu the "
                "allocation-free entry point holds per device (use pdssm_fwd with a workspace, or a longer "
                "chunk)", p.ws_bytes, (size_t)PDSSM_NOALLOC_SCRATCH_BYTES);
  if (status && ((uintptr_t)status & 3)) return fail(PDSSM_EINVAL, "status is not 4-byte aligned");
  const Sizes z = sizes(dims);
  const Range in[] = {{"u", u, z.u},         {"W_sel", W_sel, z.Wsel}, {"dict_idx", dict_idx, z.dict},
                      {"W_d", W_d, z.Wd},    {"b_d", b_d, z.bd},       {"Bu", Bu, z.Bu},
                      {"C", C, z.C},         {"h0", h0, z.h0}};
  const Range out[] = {{"k_star", k_star, z.k}, {"D", D, z.D}, {"y", y, z.y}, {"h_L", h_L, z.hL}};
  static const char* const req[] = {"u", "W_sel", "dict_idx", "W_d", "b_d", "Bu", "C", "y", "h_L", nullptr};
  if ((rc = check_ptrs(in, 8, out, 4, req))) return rc;
  for (const Range& r : in)
    if (overlap({"status", status, 4}, r)) return fail(PDSSM_EINVAL, "status overlaps input %s", r.name);
  for (const Range& r : out)
    if (overlap({"status", status, 4}, r)) return fail(PDSSM_EINVAL, "status overlaps output %s", r.name);
  void* scratch = nullptr;
  size_t cap = 0;
  hipError_t e = pdscan::noalloc_scratch(&scratch, &cap);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "device scratch lookup failed: %s", hipGetErrorString(e));
  if (p.ws_bytes > cap) return fail(PDSSM_EUNSUPPORTED, "scratch of %zu bytes < %zu needed", cap, p.ws_bytes);
  pdscan::Args a = {};
  a.p = p;
  a.u = u; a.W_sel = W_sel; a.W_d = W_d; a.b_d = b_d; a.dict = dict_idx;
  a.Bu = Bu; a.C = C; a.h0 = h0; a.k_out = k_star; a.D_out = D;
  a.y = y; a.hL = h_L; a.ws = (unsigned char*)scratch;
  if ((rc = dispatch(pdscan::kModeFused, a, stream))) return rc;
  if (status) {
    e = pdscan::launch_status(scratch, status, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return PDSSM_OK;
}

int pdssm_fwd_wb(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
                 const int32_t* dict_idx, const void* W_d, const float* b_d, const void* W_b,
                 const float* C, const float* h0, int32_t* k_star, float* D, float* y, float* h_L,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_wb_impl(dims, chunk, 1, u, W_sel, dict_idx, W_d, b_d, W_b, C, h0, k_star, D, y, h_L, workspace,
                     workspace_bytes, stream);
}

int pdssm_fwd_wb_multi(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const void* u,
                       const void* W_sel, const int32_t* dict_idx, const void* W_d, const float* b_d,
                       const void* W_b, const float* C, const float* h0, int32_t* k_star, float* D,
                       float* y, float* h_L, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_n_out(n_out);
  if (rc) return rc;
  return fwd_wb_impl(dims, chunk, n_out, u, W_sel, dict_idx, W_d, b_d, W_b, C, h0, k_star, D, y, h_L,
                     workspace, workspace_bytes, stream);
}

int pdssm_scan_fwd_pidx(const pdssm_dims* dims, int32_t chunk, const int32_t* P_idx, const float* D,
                        const float* Bu, const float* C, const float* h0, float* y, float* h_L,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!dims) return fail(PDSSM_EINVAL, "dims is NULL");
  pdssm_dims dd = *dims;
  dd.K = 1;                                        // no dictionary: one map per step
  int rc = check_dims(&dd, chunk);
  if (rc) return rc;
  Plan p;
  const int T = chunk < dd.L ? chunk : dd.L;
  // N <= 16 and chunks up to 512: the maps stream through registers (the
  // step-major scan); otherwise the step maps of a chunk are its table
  const bool sm = dd.N <= 16 && T <= 512;
  dd.K = sm ? 1 : T;
  if (!pdscan::make_plan(p, pdscan::kModeScan, dd.B, dd.H, dd.L, dd.N, dd.K, dd.d_in, dd.u_shared,
                         dd.in_dtype == PDSSM_BF16, chunk, 0, sm ? 1 : 0))
    return fail(PDSSM_EUNSUPPORTED, "chunk=%d with N=%d needs %d bytes of on-chip memory with per-step "
                "maps (limit %d); use a shorter chunk", chunk, dd.N, p.lds_bytes, pdscan::kMaxLds);
  if (lookback_giveup_hook()) {
    p.force_giveup = 1;
    p.spin_limit = 2;
  }
  if (workspace_bytes < p.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  const Sizes z = sizes(dims);
  const Range in[] = {{"P_idx", P_idx, z.D}, {"D", D, z.D}, {"Bu", Bu, z.Bu}, {"C", C, z.C},
                      {"h0", h0, z.h0}};
  const Range out[] = {{"y", y, z.y}, {"h_L", h_L, z.hL}, {"workspace", workspace, p.ws_bytes}};
  static const char* const req[] = {"P_idx", "D", "Bu", "C", "y", "h_L", "workspace", nullptr};
  if ((rc = check_ptrs(in, 5, out, 3, req))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.P_in = P_idx; a.D_in = D; a.Bu = Bu; a.C = C; a.h0 = h0;
  a.y = y; a.hL = h_L; a.ws = (unsigned char*)workspace;
  return dispatch(pdscan::kModeScan, a, stream);
}

int pdssm_scan_states(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                      const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                      const float* h0, float* y, float* h_L, float* H_all, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeScan, dims, chunk, 0, 2))) return rc;
  if (workspace_bytes < p.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                p.ws_bytes);
  const Sizes z = sizes(dims);
  const Range in[] = {{"k_star", k_star, z.k}, {"dict_idx", dict_idx, z.dict}, {"D", D, z.D},
                      {"Bu", Bu, z.Bu}, {"C", C, z.C}, {"h0", h0, z.h0}};
  const Range out[] = {{"y", y, z.y}, {"h_L", h_L, z.hL}, {"H_all", H_all, z.D},
                       {"workspace", workspace, p.ws_bytes}};
  static const char* const req[] = {"k_star", "dict_idx", "D", "Bu", "C", "y", "h_L", "H_all",
                                    "workspace", nullptr};
  if ((rc = check_ptrs(in, 6, out, 4, req))) return rc;
  pdscan::Args a = {};
  a.p = p;
  a.dict = dict_idx; a.k_in = k_star; a.D_in = D; a.Bu = Bu; a.C = C; a.h0 = h0;
  a.y = y; a.hL = h_L; a.H_all = H_all; a.ws = (unsigned char*)workspace;
  return dispatch(pdscan::kModeScan, a, stream);
}

int pdssm_scan_bwd_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  if (!bytes) return fail(PDSSM_EINVAL, "bytes is NULL");
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeScan, dims, chunk))) return rc;
  pdscan::BwdLds l;
  if (!pdscan::make_bwd_lds(p, l))
    return fail(PDSSM_EUNSUPPORTED, "chunk=%d with N=%d K=%d needs %d bytes of on-chip memory in the "
                "gradient pass (limit %d)", p.chunk, dims->N, dims->K, l.bytes, pdscan::kMaxLds);
  *bytes = pdscan::bwd_ws_bytes(p);
  return PDSSM_OK;
}

int pdssm_scan_bwd(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                   const int32_t* dict_idx, const float* D, const float* C, const float* h0,
                   const float* H_all, const float* g_y, const float* g_hL, float* g_Bu,
                   float* g_D, float* g_h0, float* g_C, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int rc = check_dims(dims, chunk);
  if (rc) return rc;
  Plan p;
  if ((rc = build_plan(p, pdscan::kModeScan, dims, chunk))) return rc;
  pdscan::BwdLds l;
  if (!pdscan::make_bwd_lds(p, l))
    return fail(PDSSM_EUNSUPPORTED, "chunk=%d with N=%d K=%d needs %d bytes of on-chip memory in the "
                "gradient pass (limit %d)", p.chunk, dims->N, dims->K, l.bytes, pdscan::kMaxLds);
  const size_t need = pdscan::bwd_ws_bytes(p);
  if (workspace_bytes < need)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  const Sizes z = sizes(dims);
  const Range in[] = {{"k_star", k_star, z.k}, {"dict_idx", dict_idx, z.dict}, {"D", D, z.D},
                      {"C", C, z.C},           {"h0", h0, z.h0},           {"H_all", H_all, z.D},
                      {"g_y", g_y, z.y},       {"g_hL", g_hL, z.hL}};
  const Range out[] = {{"g_Bu", g_Bu, z.Bu}, {"g_D", g_D, z.D},          {"g_h0", g_h0, z.h0},
                       {"g_C", g_C, z.C},    {"workspace", workspace, need}};
  static const char* const req[] = {"k_star", "dict_idx", "D", "C", "H_all", "g_y", "g_Bu",
                                    "g_D", "g_C", "workspace", nullptr};
  if ((rc = check_ptrs(in, 8, out, 5, req))) return rc;
  pdscan::BwdArgs a = {};
  a.p = p;
  a.l = l;
  a.ws_gc = pdscan::bwd_ws_gc(p);
  a.k_star = k_star; a.dict = dict_idx; a.D = D; a.C = C; a.h0 = h0; a.H_all = H_all;
  a.g_y = g_y; a.g_hL = g_hL; a.g_Bu = g_Bu; a.g_D = g_D; a.g_h0 = g_h0;
  a.ws = (unsigned char*)workspace;
  const hipError_t e = pdscan::launch_bwd(a, g_C, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

int pdssm_impulse_sens_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes) {
  pdscan::SensPlan q;
  int rc = sens_plan(q, dims, chunk);
  if (rc) return rc;
  if (!bytes) return fail(PDSSM_EINVAL, "bytes is NULL");
  *bytes = q.ws_bytes;
  return PDSSM_OK;
}

int pdssm_impulse_sens(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                       const int32_t* dict_idx, const float* D, const void* W_d, const void* W_b,
                       const float* C, const float* h0, float* dY, void* workspace,
                       size_t workspace_bytes, void* stream) {
  pdscan::SensPlan q;
  int rc = sens_plan(q, dims, chunk);
  if (rc) return rc;
  if (workspace_bytes < q.ws_bytes)
    return fail(PDSSM_EWORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, q.ws_bytes);
  const Sizes z = sizes(dims);
  const size_t ydz = (size_t)dims->B * dims->H * dims->L * dims->d_in * 4;
  const Range in[] = {{"k_star", k_star, z.k}, {"dict_idx", dict_idx, z.dict}, {"D", D, z.D},
                      {"W_d", W_d, z.Wd},      {"W_b", W_b, z.Wd},           {"C", C, z.C},
                      {"h0", h0, z.h0}};
  const Range out[] = {{"dY", dY, ydz}, {"workspace", workspace, q.ws_bytes}};
  static const char* const req[] = {"k_star", "dict_idx", "D", "W_d", "W_b", "C", "dY", "workspace",
                                    nullptr};
  if ((rc = check_ptrs(in, 7, out, 2, req))) return rc;
  pdscan::SensArgs a = {};
  a.q = q;
  a.k_star = k_star; a.dict = dict_idx; a.D = D; a.W_d = W_d; a.W_b = W_b; a.C = C; a.h0 = h0;
  a.dY = dY; a.ws = (unsigned char*)workspace;
  const hipError_t e = pdscan::launch_sens(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

int pdssm_soft_select(const pdssm_dims* dims, const void* u, const void* W_sel, const float* M,
                      const void* W_d, const float* b_d, float* M_t, int32_t* P_idx, float* D,
                      void* stream) {
  int rc = check_dims(dims, -1);
  if (rc) return rc;
  pdscan::SoftPlan q;
  if (!pdscan::make_soft_plan(q, dims->B, dims->H, dims->L, dims->N, dims->K, dims->d_in, dims->u_shared,
                              dims->in_dtype == PDSSM_BF16))
    return fail(PDSSM_EUNSUPPORTED, "soft selection: N=%d K=%d d_in=%d (N, K at most %d, %d; d_in one of "
                "16, 32, 64, 128)", dims->N, dims->K, dims->d_in, pdscan::kSoftMaxN, pdscan::kSoftMaxK);
  const Sizes z = sizes(dims);
  const size_t mz = (size_t)dims->H * dims->K * dims->N * dims->N * 4;
  const size_t mtz = (size_t)dims->B * dims->H * dims->L * dims->N * dims->N * 4;
  const Range in[] = {{"u", u, z.u}, {"W_sel", W_sel, z.Wsel}, {"M", M, mz}, {"W_d", W_d, z.Wd},
                      {"b_d", b_d, z.bd}};
  const Range out[] = {{"M_t", M_t, mtz}, {"P_idx", P_idx, z.D}, {"D", D, z.D}};
  static const char* const req[] = {"u", "W_sel", "M", "W_d", "b_d", "M_t", "P_idx", "D", nullptr};
  if ((rc = check_ptrs(in, 5, out, 3, req))) return rc;
  pdscan::SoftArgs a = {};
  a.q = q;
  a.u = u; a.W_sel = W_sel; a.M = M; a.W_d = W_d; a.b_d = b_d; a.M_t = M_t; a.P_idx = P_idx; a.D = D;
  const hipError_t e = pdscan::launch_soft(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

int pdssm_dict_hardmax(int32_t H, int32_t K, int32_t N, const float* M, int32_t* dict_idx, void* stream) {
  if (H < 1 || K < 1 || N < 1) return fail(PDSSM_EINVAL, "H, K, N must be >= 1 (got %d %d %d)", H, K, N);
  if (N > 64) return fail(PDSSM_EUNSUPPORTED, "N=%d > 64", N);
  const size_t mz = (size_t)H * K * N * N * 4, dz = (size_t)H * K * N * 4;
  const Range in[] = {{"M", M, mz}};
  const Range out[] = {{"dict_idx", dict_idx, dz}};
  static const char* const req[] = {"M", "dict_idx", nullptr};
  int rc = check_ptrs(in, 1, out, 1, req);
  if (rc) return rc;
  const hipError_t e = pdscan::launch_dict_hardmax(M, dict_idx, H * K, N, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PDSSM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return PDSSM_OK;
}

}  // extern "C"

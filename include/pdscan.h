/*
 * libpdscan -- hard-selection PD-SSM forward pass for AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no C++ or framework types.
 *
 * What is computed (per batch element b, head h, step t):
 *   scores  s_t[k] = sum_c W_sel[h,k,c] u_t[c]                 (k < K)
 *   select  k*_t   = lowest k with s_t[k] = max_j s_t[j]
 *   diag    D_t[n] = 1 / (1 + exp(-(sum_c W_d[h,n,c] u_t[c] + b_d[h,n])))
 *   step    h_t[i] = Bu_t[i] + sum_{j : dict[h,k*_t,j] = i} D_t[j] h_{t-1}[j]
 *   output  y_t    = sum_i C[h,i] h_t[i]
 * with h_{-1} = h0 and h_L the state after the last step.
 *
 * Sources: "Flash PD-SSM: Memory-Optimized Structured Sparse State-Space
 * Models" (gist.science explainer), technical summary -- methodology item 1
 * (scores from a linear map of u_t, argmax over a precomputed dictionary of K
 * sparse matrices, the chosen matrix a one-hot column selector, O(LN) memory)
 * and item 3 (three-phase chunked kernel: per-chunk sequential recurrences,
 * an inter-chunk prefix scan of carry states, a carry correction).  Readings
 * where the pages are silent: column j of the selected matrix carries its one
 * in row dict[h,k*,j]; the transition is that selector times diag(D_t); D_t
 * is the logistic of a second linear map; Bu is supplied by the caller; C has
 * one output per head.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a caller-owned DEVICE pointer, row-major and
 *     contiguous, 16-byte aligned.  Shapes are given below in brackets.
 *   - u, W_sel and W_d are fp32 (dims.in_dtype = PDSSM_F32) or bf16
 *     (PDSSM_BF16, stored as raw 16-bit words).  Everything else is fp32
 *     (int32 for indices).
 *   - u is [B,H,L,d_in] when dims.u_shared = 0, or [B,L,d_in] shared by all
 *     heads when dims.u_shared = 1.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  PDSSM_OK means "enqueued".  Faults surface at the caller's
 *     next synchronisation.
 *   - The library allocates nothing, never synchronises the device and holds
 *     no global mutable state: scratch memory comes from the caller's
 *     workspace.  Two calls that share one workspace must be ordered on one
 *     stream.
 *   - Workspace header.  Every call that takes a workspace clears it first;
 *     its 32-bit word at byte offset 4 is then nonzero when a look-back wait
 *     of that call (the inter-chunk carry, phase B) gave up after about 4M
 *     window reads.  The affected chunks then continued from the zero carry
 *     (h0 in the forward scans), so y, h_L and every gradient or sensitivity
 *     output of that call are wrong.  A wait ends only when the preceding
 *     chunks have published, which every launch order the runtime uses
 *     guarantees; the word guards against a stalled device.  Read it with
 *     pdssm_workspace_status after the call, on the same stream.
 *     (Test hook: with PDSSM_TEST_LOOKBACK_GIVEUP=1 in the environment every
 *     wait ignores the carries it finds and gives up after two reads, so a
 *     test can set the word on purpose.  Never set it in normal use.)
 *   - Tuning hook: PDSSM_XCD_HEAD_GROUPS = 0, 1, 2, 4 or 8 in the environment
 *     overrides how the general fused kernel groups its (b, h) sequences
 *     over the eight dies (0: no grouping).  Results do not depend on it.
 *   - Arguments are validated on the host before any HIP call.  On failure
 *     nothing is enqueued and a negative pdssm_status is returned; the
 *     calling thread's pdssm_last_error() then describes the problem.
 *   - Preconditions NOT checked on the device: dict values lie in [0, N);
 *     inputs are finite.
 *   - Shape limits (else PDSSM_EUNSUPPORTED): 1 <= N <= 64, 1 <= K <= 64,
 *     K + N <= 128, d_in % 8 == 0, d_in <= 8192, and the per-chunk on-chip
 *     footprint (about chunk * (N + 2) * 4 bytes) within 64 KiB (the folded
 *     and multi-output calls on the general kernel: within 160 KiB, see
 *     pdssm_fwd_wb).
 */
#ifndef PDSCAN_H
#define PDSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PDSSM_ABI_VERSION 1

typedef enum {
  PDSSM_OK = 0,
  PDSSM_EINVAL = -1,        /* bad argument: NULL, size <= 0, misaligned, aliasing */
  PDSSM_EUNSUPPORTED = -2,  /* valid but outside the shape limits above           */
  PDSSM_EWORKSPACE = -3,    /* workspace smaller than the matching *_workspace_bytes */
  PDSSM_EHIP = -4           /* a HIP launch or runtime call failed                */
} pdssm_status;

typedef enum { PDSSM_F32 = 0, PDSSM_BF16 = 1 } pdssm_dtype;

typedef struct {
  int32_t B, H, L, N, K, d_in;
  int32_t u_shared; /* 0: u is [B,H,L,d_in]; 1: u is [B,L,d_in], read by every head */
  int32_t in_dtype; /* pdssm_dtype of u, W_sel and W_d                               */
} pdssm_dims;

/* Selection: scores, argmax and the logistic diagonal for every (b,h,t)
 * ("Flash PD-SSM" summary, Methodology 1: fp32 scores over the K dictionary
 * entries, the argmax with ties to the lowest index, D = sigmoid(W_d u + b_d)).
 *   u [B,H,L,d] | [B,L,d]; W_sel [H,K,d]; W_d [H,N,d]; b_d [H,N]
 *   k_star [B,H,L] int32 (out, required); D [B,H,L,N] fp32 (out, required)
 *   dict_idx [H,K,N] int32 and P_idx [B,H,L,N] int32: optional pair.  When
 *   P_idx is non-NULL it receives dict_idx[h, k*_t, :] (the selected matrix as
 *   its N row indices) and dict_idx must be non-NULL; otherwise both may be
 *   NULL.
 * Score GEMMs run as fp32 MFMA for fp32 inputs and for bf16 inputs with
 * d_in < 128 (bf16 products are exact in fp32), and as bf16 MFMA with fp32
 * accumulation for bf16 inputs with d_in >= 128.  With u shared by the heads
 * in bf16 (K <= 32, N <= 64 a multiple of 4, d_in a multiple of 64, B*L below
 * 2^31) the selection runs as one bf16 GEMM over all tokens and heads (the
 * heads of each 256-token tile on one die, so the tile is read from HBM once). */
int pdssm_select(const pdssm_dims* dims, const void* u, const void* W_sel,
                 const int32_t* dict_idx, const void* W_d, const float* b_d,
                 int32_t* k_star, float* D, int32_t* P_idx, void* stream);

/* Bytes of workspace pdssm_scan_fwd needs for these dims and chunk length. */
int pdssm_scan_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes);

/* Chunked scan given selections: phases A, B and C.
 *   k_star [B,H,L] int32; dict_idx [H,K,N] int32; D [B,H,L,N]; Bu [B,H,L,N];
 *   C [H,N]; h0 [B,H,N] or NULL (zero state)
 *   y [B,H,L] (out); h_L [B,H,N] (out)
 *   chunk >= 1: steps per chunk (the last chunk may be shorter).  Results do
 *   not depend on chunk beyond floating-point rounding.
 *   workspace: device scratch of at least pdssm_scan_workspace_bytes bytes;
 *   its contents on entry do not matter. */
int pdssm_scan_fwd(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                   const int32_t* dict_idx, const float* D, const float* Bu,
                   const float* C, const float* h0, float* y, float* h_L,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pdssm_fwd needs for these dims and chunk length.  For
 * the shapes pdssm_fwd runs as two passes (below) this includes room for k*
 * and D: B*H*L*(N+1)*4 bytes beyond the look-back words. */
int pdssm_fwd_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes);

/* Selection + chunked scan.  Arguments as in pdssm_select and
 * pdssm_scan_fwd; k_star [B,H,L] and D [B,H,L,N] are optional outputs (NULL:
 * not written).
 * Passes.  One fused kernel reads u and Bu once, except for u shared by the
 * heads with N > 32 and the shapes of pdssm_select's all-heads GEMM: there
 * the GEMM writes k* and D (into the caller's outputs, or the workspace) and
 * the chunked scan of pdssm_scan_fwd reads them, on the same stream.  Results
 * agree to the tolerances of both paths (k* identical; y and h_L differ by
 * rounding order only).
 * Score precision.  fp32 inputs on the step-major kernel (per-head u, N <= 16,
 * K <= 16, d_in in {32, 64}) form every product on the bf16 matrix cores from
 * an exact three-piece split of each fp32 operand (x = x0 + x1 + x2, each
 * piece the next eight significant bits), keeping the six piece products
 * whose weight is at least 2^-16 of |x w| and accumulating in fp32: the
 * dropped terms are below 2^-23 |x w|, so the scores carry fp32 accuracy.
 * Other fp32 shapes use fp32 MFMA; bf16 inputs use bf16 MFMA (d_in >= 128)
 * or exact fp32 MFMA products (d_in < 128). */
int pdssm_fwd(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
              const int32_t* dict_idx, const void* W_d, const float* b_d,
              const float* Bu, const float* C, const float* h0,
              int32_t* k_star, float* D, float* y, float* h_L,
              void* workspace, size_t workspace_bytes, void* stream);

/* Look-back scratch the allocation-free call below holds on each device. */
#define PDSSM_NOALLOC_SCRATCH_BYTES (16u << 20)

/* pdssm_fwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments and outputs as in pdssm_fwd, always on the
 * single fused kernel (never the two-pass route, whose k* and D would need
 * room); its look-back scratch lives in a 16 MiB device array that the
 * library holds on each GPU it runs on, until the process ends.
 *   status: optional (NULL: not written); one uint32 in device memory or
 *     pinned host memory, 4-byte aligned.  The call ORs its look-back error
 *     word into status[0] (nonzero = a wait gave up; see "Workspace header").
 * Every call on a GPU uses that GPU's one array (the array of the device
 * current at the call): two calls that may overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results;
 * order them on one stream.  Each call clears the part of the array it uses
 * first, so nothing carries over from the previous call.  The array is found
 * on the first call on each device; calls allocate nothing.
 * Returns PDSSM_EUNSUPPORTED when the call needs more scratch than
 * PDSSM_NOALLOC_SCRATCH_BYTES (the fused kernel's look-back words above 16
 * MiB), with the other statuses as pdssm_fwd. */
int pdssm_fwd_noalloc(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
                      const int32_t* dict_idx, const void* W_d, const float* b_d,
                      const float* Bu, const float* C, const float* h0,
                      int32_t* k_star, float* D, float* y, float* h_L,
                      uint32_t* status, void* stream);

/* pdssm_fwd with the drive term computed in the same pass: Bu_t = W_b u_t
 * (the input map B of the state-space recurrence, "Flash PD-SSM" summary,
 * problem statement and methodology item 1) is a third set of columns of the
 * selection GEMM, so Bu is never read from or written to memory.
 *   W_b [H,N,d_in] (in, u's dtype): row n holds the weights of state row n.
 *   All other arguments, the workspace (pdssm_fwd_workspace_bytes) and the
 *   outputs as in pdssm_fwd (u per head or shared by the heads).  The
 *   products are formed like the scores (fp32 for fp32 inputs, bf16 x bf16
 *   with fp32 accumulation for bf16 inputs with d_in >= 128).
 * Shapes: the step-major kernel (per-head u, N <= 16, K <= 16, chunk <= 512,
 * fp32 d_in in {16, 32, 64} or bf16 d_in = 128: W_b is a third MFMA tile) and
 * the general kernel (every other shape: the drive terms of a chunk go to an
 * on-chip [N][chunk] buffer) when its selection GEMM holds the columns:
 * K + 2N <= 128, or for bf16 inputs with d_in >= 256 (a multiple of 32)
 * ceil(K/16) + 2 ceil(N/16) <= 10 tiles (N = 64 with K <= 32).  On the
 * general kernel the chunk's on-chip footprint (about chunk * (2N + 2) * 4
 * bytes plus the dictionary tables) may take up to the 160 KiB LDS of one
 * compute unit.  Anything else returns PDSSM_EUNSUPPORTED.
 * Exception: u shared by the heads in bf16 with N > 32 (the shapes of
 * pdssm_fwd's two passes) runs the all-heads selection GEMM, a second GEMM of
 * the same tiles that writes Bu = W_b u into the workspace, then the chunked
 * scan (pdssm_scan_fwd_multi with n_out rows): Bu passes through memory
 * there, and the on-chip limit above does not apply. */
int pdssm_fwd_wb(const pdssm_dims* dims, int32_t chunk, const void* u, const void* W_sel,
                 const int32_t* dict_idx, const void* W_d, const float* b_d,
                 const void* W_b, const float* C, const float* h0,
                 int32_t* k_star, float* D, float* y, float* h_L,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Chunked scan that also writes the state after every step.
 *   Arguments as in pdssm_scan_fwd (same workspace size), plus
 *   H_all [B,H,L,N] (out): h_t for t = 0..L-1, the states the gradient pass
 *   below reads.  Each lane group replays its sub-chunk from its true entering
 *   state, so y here is the sequential recurrence itself. */
int pdssm_scan_states(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                      const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                      const float* h0, float* y, float* h_L, float* H_all, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of workspace pdssm_scan_bwd needs for these dims and chunk length
 * (PDSSM_EUNSUPPORTED when its on-chip layout, about chunk * N * 4 bytes
 * plus the dictionary, exceeds 64 KiB). */
int pdssm_scan_bwd_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes);

/* Gradient of a scalar loss through the scan for fixed selections
 * ("Flash PD-SSM" summary, methodology item 2 covers the selection's own
 * surrogate gradient, which is not computed here: k* carries no gradient).
 * Given dLoss/dy and dLoss/dh_L, the adjoint recurrence
 *   lam_{L-1} = C g_y[L-1] + g_hL,  lam_t = C g_y[t] + A_{t+1}^T lam_{t+1}
 * gives
 *   g_Bu [B,H,L,N] = lam_t                              (out, required)
 *   g_D  [B,H,L,N] = lam_t[dict[h,k*_t,j]] h_{t-1}[j]   (out, required)
 *   g_h0 [B,H,N]   = A_0^T lam_0                        (out, optional)
 *   g_C  [H,N]     = sum over b and t of g_y h_t        (out, required)
 * Inputs: k_star, dict_idx, D, C and h0 (NULL = zero) as in the forward
 * call; H_all [B,H,L,N] the forward states (pdssm_scan_states); g_y [B,H,L];
 * g_hL [B,H,N] or NULL (zero).  chunk: as in the forward scan.  g_C is summed
 * in a fixed order, so results are bit-identical from run to run. */
int pdssm_scan_bwd(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                   const int32_t* dict_idx, const float* D, const float* C, const float* h0,
                   const float* H_all, const float* g_y, const float* g_hL, float* g_Bu,
                   float* g_D, float* g_h0, float* g_C, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Several outputs per head: y_t = C h_t ("Flash PD-SSM" summary, methodology
 * item 1) with C holding n_out rows per head, the output channels of a layer
 * that reads u and writes y.  The pass of pdssm_fwd_wb with
 *   n_out  1 <= n_out <= 4 (else PDSSM_EINVAL);
 *   C      [H,n_out,N] fp32 (in): row o of head h is C[h,o,:];
 *   y      [B,H,L,n_out] fp32 (out): y[b,h,t,o] = C[h,o,:] . h_t.
 * Everything else, the workspace (pdssm_fwd_workspace_bytes) and the shape
 * limits as in pdssm_fwd_wb.  The on-chip output weights grow with n_out
 * (n_out * N * chunk * 4 bytes), so the longest chunk shrinks with it
 * (step-major kernel, N = 16: n_out = 2 up to chunk 256, n_out = 3 or 4 up to
 * 128; general kernel within 160 KiB, e.g. N = 64 with d_in = 768 and the
 * drive folded: n_out = 2 up to chunk 128); a chunk that does not fit returns
 * PDSSM_EUNSUPPORTED. */
int pdssm_fwd_wb_multi(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const void* u,
                       const void* W_sel, const int32_t* dict_idx, const void* W_d, const float* b_d,
                       const void* W_b, const float* C, const float* h0, int32_t* k_star, float* D,
                       float* y, float* h_L, void* workspace, size_t workspace_bytes, void* stream);

/* pdssm_scan_fwd with several outputs per head: C [H,n_out,N] and
 * y [B,H,L,n_out] as in pdssm_fwd_wb_multi; 1 <= n_out <= 4.  The step-major
 * scan (N <= 16, K <= 16, chunk <= 512) or the general one; a chunk whose
 * per-output on-chip rows do not fit returns PDSSM_EUNSUPPORTED.  Workspace
 * as pdssm_scan_workspace_bytes. */
int pdssm_scan_fwd_multi(const pdssm_dims* dims, int32_t chunk, int32_t n_out, const int32_t* k_star,
                         const int32_t* dict_idx, const float* D, const float* Bu, const float* C,
                         const float* h0, float* y, float* h_L, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of workspace pdssm_impulse_sens needs for these dims and chunk length
 * (256 + nC * B * H * 4 * N * 8 bytes: per chunk, its composed PD map and the
 * inclusive map entering the next chunk, 2 N tagged words each; no tangent
 * state crosses a chunk). */
int pdssm_impulse_sens_workspace_bytes(const pdssm_dims* dims, int32_t chunk, size_t* bytes);

/* Sensitivity of every output to the first input, dY[b,h,t,:] = dy_t / du_0,
 * for fixed selections ("Breaking the Memory Wall: Exact Analytical
 * Differentiation via Tiled Operator-Space Evolution" summary: exact
 * derivatives over long sequences without storing the graph; here the
 * 128k-step impulse-response derivative of this layer).  u_0 enters step 0
 * through D_0 = sigmoid(W_d u_0 + b_d) and the drive W_b u_0, so the state
 * tangent after step 0 is J = W_b + P_0 diag(D_0 (1 - D_0) h0) W_d, and
 * dY_t = C A_t ... A_1 J (k*_0 carries no derivative).
 *   k_star [B,H,L], dict_idx [H,K,N], D [B,H,L,N] (in): the selections of a
 *     forward pass (pdssm_select, or pdssm_fwd's optional outputs).
 *   W_d, W_b [H,N,d_in] (in, dtype in_dtype); C [H,N]; h0 [B,H,N] or NULL.
 *   dY [B,H,L,d_in] fp32 (out).
 * Shapes: per-head layout, N <= 16, d_in a multiple of 16 and at most 128,
 * on-chip layout within 64 KiB (chunk <= 512); else PDSSM_EUNSUPPORTED. */
int pdssm_impulse_sens(const pdssm_dims* dims, int32_t chunk, const int32_t* k_star,
                       const int32_t* dict_idx, const float* D, const void* W_d, const void* W_b,
                       const float* C, const float* h0, float* dY, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The scan of pdssm_scan_fwd on per-step column maps instead of a
 * dictionary and selections: P_idx [B,H,L,N] (in) holds, for every step, the
 * row of column j's one (as pdssm_soft_select or pdssm_select's P_idx write
 * it; values in [0, N)).  dims->K is ignored.  Workspace as
 * pdssm_scan_workspace_bytes.  With N <= 16 and chunk <= 512 the maps stream
 * through registers; otherwise an on-chip table holds one map per step of a
 * chunk (chunk * (N + 1) * 8 bytes), and a chunk whose table does not fit
 * (N = 16: above 512; N = 20: above 548) returns PDSSM_EUNSUPPORTED. */
int pdssm_scan_fwd_pidx(const pdssm_dims* dims, int32_t chunk, const int32_t* P_idx, const float* D,
                        const float* Bu, const float* C, const float* h0, float* y, float* h_L,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Selection of the original (soft-selection) PD-SSM, kept as a comparison
 * path ("Flash PD-SSM" summary, background: the original model mixes dense
 * dictionary matrices and sparsifies the mixture column by column, at
 * O(L N^2) memory).  Per step t of sequence (b, h):
 *   alpha_t = softmax(W_sel u_t), M_t = sum_k alpha_t[k] M[h,k]  (written to M_t),
 *   P_idx_t[j] = lowest row i with M_t[i, j] maximal (column hardmax),
 *   D_t = sigmoid(W_d u_t + b_d).
 *   u, W_sel, W_d, b_d as in pdssm_select (fp32 or bf16); M [H,K,N,N] fp32,
 *   M[h,k,i,j] = row i, column j.  Outputs: M_t [B,H,L,N,N], P_idx [B,H,L,N],
 *   D [B,H,L,N] (all required).  fp32 arithmetic.
 * Shapes: N <= 16, K <= 16, d_in in {16, 32, 64, 128}; else PDSSM_EUNSUPPORTED. */
int pdssm_soft_select(const pdssm_dims* dims, const void* u, const void* W_sel, const float* M,
                      const void* W_d, const float* b_d, float* M_t, int32_t* P_idx, float* D,
                      void* stream);

/* The sparse dictionary of the hard-selection path from dense parameters:
 * dict_idx[h,k,j] = lowest row i with M[h,k,i,j] maximal (column hardmax of
 * every dictionary matrix; "Flash PD-SSM" summary, methodology item 1).
 *   M [H,K,N,N] fp32 (in); dict_idx [H,K,N] int32 (out). */
int pdssm_dict_hardmax(int32_t H, int32_t K, int32_t N, const float* M, int32_t* dict_idx, void* stream);

/* Static text for a status code. */
const char* pdssm_status_str(int status);

/* Description of the calling thread's most recent failure ("" if none). */
const char* pdssm_last_error(void);

/* PDSSM_ABI_VERSION of the loaded library. */
int pdssm_abi_version(void);

/* Look-back status of the most recent call on `workspace` (any of the calls
 * above that take a workspace): enqueues on `stream` a one-lane kernel that
 * ORs the workspace error word (see "Workspace header" above; nonzero = some
 * look-back wait of that call gave up and its outputs are wrong) into
 * status[0].  Order it after the call on the same stream and read status
 * after synchronising; zero status[0] first, or keep ORing the words of
 * several calls into it to check them all at once.
 *   workspace: the call's workspace (16-byte aligned, at least 256 bytes).
 *   status: one uint32 in device memory or in pinned host memory visible to
 *     the device (4-byte aligned); owned by the caller.
 * Returns PDSSM_EINVAL for NULL or misaligned pointers, PDSSM_EWORKSPACE for
 * fewer than 256 bytes. */
int pdssm_workspace_status(const void* workspace, size_t workspace_bytes, uint32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDSCAN_H */

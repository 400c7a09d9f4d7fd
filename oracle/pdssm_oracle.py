"""fp64 CPU oracle for the hard-selection PD-SSM forward pass.

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it, and this module imports nothing from
the product path.

It is the plain definition, written out slowly:

* selection -- "Flash PD-SSM: Memory-Optimized Structured Sparse State-Space
  Models" (gist.science explainer), technical summary, methodology item 1
  (hard selection): a linear map of u_t gives K scores, the highest-scoring
  precomputed sparse matrix is taken (argmax) and used as is.  Ties go to the
  lowest index (numpy's argmax returns the first maximum).
* the selected matrix is a one-hot column selector (same item, complexity
  paragraph).  Reading: P[idx[j], j] = 1, i.e. column j carries its one in
  row idx[j]; the transition is A_t = P^(k*) D_t with the diagonal
  D_t = sigmoid(W_d u_t + b_d) scaling column j before it moves.
* the recurrence of a linear SSM (problem statement of the same summary):
  h_t = A_t h_{t-1} + Bu_t, y_t = C h_t, with h0 the state before step 0,
  y_t read after the update and h_L the state after the last step.

Everything is upcast exactly to fp64 first.  ``scan`` builds the dense N x N
transition of every step and multiplies; it never uses the sparse structure.

``forward_wb`` is the same forward pass with the drive terms Bu_t = W_b u_t
formed from the input (``drive``) instead of being given; ``scan_multi`` /
``forward_wb_multi`` read several outputs per head, y_t = C h_t with C
holding n_out rows, from the states of ``scan_states``.

``soft_select`` / ``scan_pidx`` are the original soft-selection model, kept
as a comparison path: a softmax-weighted mixture of dense dictionary
matrices, its column hardmax per step, and the recurrence on those per-step
maps; ``dict_hardmax`` builds the sparse dictionary from dense matrices.

``impulse_sensitivity`` is dy_t / du_0 for fixed selections, carried forward
from step 0 by the same dense transitions (forward mode).

``scan_vjp`` is the gradient of a scalar loss through that recurrence for
fixed selections (the adjoint recurrence with the dense transposed
transitions); ``scan_states`` returns the state after every step, which the
gradient with respect to the diagonal needs.

``three_phase`` is a separate fp64 evaluation that follows the pages' kernel
description (same summary, methodology item 3: phase A runs independent
sequential recurrences inside chunks, phase B prefix-scans the chunk
summaries into carry states, phase C applies the carry corrections), with
dense matrices.  It exists so that the chunked identity can be checked against
``scan``.  ``pd_compose`` / ``pd_apply`` state the O(N) algebra of these maps
(composition by an index gather and a scale product, application by a
scatter-add) so that it can be checked against dense products.
"""

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def sigmoid(z):
    """Logistic function 1 / (1 + exp(-z)) in fp64."""
    z = np.asarray(z, dtype=F64)
    return 1.0 / (1.0 + np.exp(-z))


def scores(u, W, u_shared):
    """Linear forms of every input row: out[b,h,t,k] = sum_c W[h,k,c] u[b,(h),t,c].

    u: [B,H,L,d] (per head) or [B,L,d] (shared by all heads); W: [H,M,d].
    Returns fp64 [B,H,L,M]."""
    u = np.asarray(u, dtype=F64)
    W = np.asarray(W, dtype=F64)
    if u_shared:
        # [B,1,L,d] @ [1,H,d,M]
        return np.matmul(u[:, None], np.swapaxes(W, -1, -2)[None])
    return np.matmul(u, np.swapaxes(W, -1, -2)[None])


def select(u, W_sel, W_d, b_d, u_shared=False):
    """Hard selection and input-dependent diagonal.

    Returns (k_star int32 [B,H,L], D fp64 [B,H,L,N], s fp64 [B,H,L,K])."""
    s = scores(u, W_sel, u_shared)
    # the decision is taken on the scores rounded to fp32: the pages fix no
    # precision for the scores, and fp32 is the one the kernel decides in;
    # the first maximum wins
    k_star = np.argmax(s.astype(np.float32), axis=-1).astype(np.int32)
    z = scores(u, W_d, u_shared) + np.asarray(b_d, dtype=F64)[None, :, None, :]
    return k_star, sigmoid(z), s


# --------------------------------------------------------------------------
# transitions and the sequential scan
# --------------------------------------------------------------------------

def transition_matrix(idx, dvals):
    """Dense A = P D for one map: A[..., idx[j], j] = dvals[j], zeros elsewhere.

    idx: int [..., N]; dvals: [..., N].  Returns fp64 [..., N, N]."""
    idx = np.asarray(idx)
    dvals = np.asarray(dvals, dtype=F64)
    N = idx.shape[-1]
    lead = idx.shape[:-1]
    A = np.zeros(lead + (N, N), dtype=F64)
    flat_idx = idx.reshape(-1, N)
    flat_d = dvals.reshape(-1, N)
    Af = A.reshape(-1, N, N)
    cols = np.arange(N)
    for r in range(flat_idx.shape[0]):
        Af[r, flat_idx[r], cols] = flat_d[r]
    return A


def scan(k_star, dict_idx, D, Bu, C, h0=None):
    """Sequential recurrence with dense transitions.

    k_star [B,H,L] int; dict_idx [H,K,N] int; D [B,H,L,N]; Bu [B,H,L,N];
    C [H,N]; h0 [B,H,N] or None (zeros).  Returns (y fp64 [B,H,L],
    h_L fp64 [B,H,N])."""
    k_star = np.asarray(k_star)
    dict_idx = np.asarray(dict_idx)
    D = np.asarray(D, dtype=F64)
    Bu = np.asarray(Bu, dtype=F64)
    C = np.asarray(C, dtype=F64)
    B, H, L = k_star.shape
    N = dict_idx.shape[-1]
    x = np.zeros((B, H, N), dtype=F64) if h0 is None else np.array(h0, dtype=F64)
    y = np.zeros((B, H, L), dtype=F64)
    heads = np.arange(H)[None, :]
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    cols = np.arange(N)[None, None, :]
    for t in range(L):
        rows = dict_idx[heads, k_star[:, :, t]]            # [B,H,N]: row of column j
        A = np.zeros((B, H, N, N), dtype=F64)
        A[bi, hi, rows, cols] = D[:, :, t]
        x = np.matmul(A, x[..., None])[..., 0] + Bu[:, :, t]
        y[:, :, t] = (C[None] * x).sum(-1)
    return y, x


def scan_states(k_star, dict_idx, D, Bu, h0=None):
    """The state after every step of ``scan``'s recurrence, fp64 [B,H,L,N]
    (h_t for t = 0..L-1; h_{L-1} is h_L)."""
    k_star = np.asarray(k_star)
    dict_idx = np.asarray(dict_idx)
    D = np.asarray(D, dtype=F64)
    Bu = np.asarray(Bu, dtype=F64)
    B, H, L = k_star.shape
    N = dict_idx.shape[-1]
    x = np.zeros((B, H, N), dtype=F64) if h0 is None else np.array(h0, dtype=F64)
    out = np.zeros((B, H, L, N), dtype=F64)
    heads = np.arange(H)[None, :]
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    cols = np.arange(N)[None, None, :]
    for t in range(L):
        rows = dict_idx[heads, k_star[:, :, t]]
        A = np.zeros((B, H, N, N), dtype=F64)
        A[bi, hi, rows, cols] = D[:, :, t]
        x = np.matmul(A, x[..., None])[..., 0] + Bu[:, :, t]
        out[:, :, t] = x
    return out


def scan_vjp(k_star, dict_idx, D, Bu, C, h0, g_y, g_hL=None):
    """Gradient of a scalar loss through ``scan`` for fixed selections.

    Given g_y = dLoss/dy [B,H,L] and g_hL = dLoss/dh_L [B,H,N] (None: zero),
    returns dLoss/d(Bu, D, h0, C) as fp64 arrays [B,H,L,N], [B,H,L,N],
    [B,H,N], [H,N].  The selections k* are held fixed: the argmax has no
    derivative, and the pages' surrogate for it ("Flash PD-SSM" summary,
    methodology item 2, straight-through estimator) is not part of this.

    The adjoint recurrence of h_t = A_t h_{t-1} + Bu_t, y_t = C h_t, run
    backwards with the dense transposed transitions:
        lam_{L-1} = C^T g_y[L-1] + g_hL,
        lam_t     = C^T g_y[t] + A_{t+1}^T lam_{t+1},
    and then dBu_t = lam_t, dA_t = lam_t h_{t-1}^T (read at the entries
    A_t[idx[j], j] = D_t[j]), dh0 = A_0^T lam_0, dC = sum_{b,t} g_y h_t^T."""
    k_star = np.asarray(k_star)
    dict_idx = np.asarray(dict_idx)
    D = np.asarray(D, dtype=F64)
    C = np.asarray(C, dtype=F64)
    g_y = np.asarray(g_y, dtype=F64)
    B, H, L = k_star.shape
    N = dict_idx.shape[-1]
    h0f = np.zeros((B, H, N), dtype=F64) if h0 is None else np.array(h0, dtype=F64)
    states = scan_states(k_star, dict_idx, D, Bu, h0f)
    lam = np.zeros((B, H, N), dtype=F64) if g_hL is None else np.array(g_hL, dtype=F64)
    g_Bu = np.zeros((B, H, L, N), dtype=F64)
    g_D = np.zeros((B, H, L, N), dtype=F64)
    heads = np.arange(H)[None, :]
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    cols = np.arange(N)[None, None, :]
    for t in range(L - 1, -1, -1):
        lam = lam + C[None] * g_y[:, :, t, None]
        g_Bu[:, :, t] = lam
        rows = dict_idx[heads, k_star[:, :, t]]
        A = np.zeros((B, H, N, N), dtype=F64)
        A[bi, hi, rows, cols] = D[:, :, t]
        h_prev = states[:, :, t - 1] if t > 0 else h0f
        dA = lam[..., :, None] * h_prev[..., None, :]       # [B,H,N,N]
        g_D[:, :, t] = dA[bi, hi, rows, cols]
        lam = np.matmul(np.swapaxes(A, -1, -2), lam[..., None])[..., 0]
    g_h0 = lam
    g_C = np.einsum("bhl,bhln->hn", g_y, states)
    return g_Bu, g_D, g_h0, g_C


def dict_hardmax(M):
    """Column hardmax of every dense dictionary matrix: out[h,k,j] = the
    lowest row i with M[h,k,i,j] maximal (numpy's argmax returns the first
    maximum).  M [H,K,N,N] (row i, column j) -> int [H,K,N]."""
    return np.argmax(np.asarray(M, dtype=F64), axis=-2)


def soft_select(u, W_sel, M, W_d, b_d, u_shared=False):
    """Selection of the original soft-selection PD-SSM ("Flash PD-SSM"
    summary, background): alpha_t = softmax(W_sel u_t) over the K dense
    dictionary matrices, the convex combination M_t = sum_k alpha_t[k] M[h,k],
    its column hardmax P_idx_t[j] = lowest row i with M_t[i, j] maximal, and
    D_t = sigmoid(W_d u_t + b_d).  fp64.

    Returns dict(alpha [B,H,L,K], M_t [B,H,L,N,N], P_idx [B,H,L,N],
    gap [B,H,L,N] (top minus runner-up of every column), D [B,H,L,N])."""
    s = scores(u, W_sel, u_shared)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    alpha = e / e.sum(axis=-1, keepdims=True)
    Mt = np.einsum("bhlk,hkij->bhlij", alpha, np.asarray(M, dtype=F64))
    P_idx = np.argmax(Mt, axis=-2)
    srt = np.sort(Mt, axis=-2)
    gap = srt[..., -1, :] - srt[..., -2, :] if Mt.shape[-2] > 1 else np.full(P_idx.shape, np.inf)
    D = sigmoid(scores(u, W_d, u_shared) + np.asarray(b_d, dtype=F64)[None, :, None, :])
    return {"alpha": alpha, "M_t": Mt, "P_idx": P_idx, "gap": gap, "D": D}


def scan_pidx(P_idx, D, Bu, C, h0=None):
    """The sequential recurrence on per-step column maps: A_t[P_idx_t[j], j] =
    D_t[j], dense, fp64.  P_idx [B,H,L,N].  Returns (y [B,H,L], h_L [B,H,N])."""
    P_idx = np.asarray(P_idx)
    D = np.asarray(D, dtype=F64)
    Bu = np.asarray(Bu, dtype=F64)
    C = np.asarray(C, dtype=F64)
    B, H, L, N = P_idx.shape
    x = np.zeros((B, H, N), dtype=F64) if h0 is None else np.array(h0, dtype=F64)
    y = np.zeros((B, H, L), dtype=F64)
    bi = np.arange(B)[:, None, None]
    hi = np.arange(H)[None, :, None]
    cols = np.arange(N)[None, None, :]
    for t in range(L):
        A = np.zeros((B, H, N, N), dtype=F64)
        A[bi, hi, P_idx[:, :, t], cols] = D[:, :, t]
        x = np.matmul(A, x[..., None])[..., 0] + Bu[:, :, t]
        y[:, :, t] = (C[None] * x).sum(-1)
    return y, x


def impulse_sensitivity(k_star, dict_idx, D, W_d, W_b, C, h0=None):
    """Sensitivity of every output to the first input, dy_t / du_0, for fixed
    selections (the impulse-response derivative of "Breaking the Memory Wall:
    Exact Analytical Differentiation via Tiled Operator-Space Evolution",
    abstract: exact derivatives of an SSM over a long sequence).

    u_0 enters only step 0: through the diagonal D_0 = sigmoid(W_d u_0 + b_d),
    whose derivative is D_0 (1 - D_0) W_d, and through the drive W_b u_0 (k*_0
    is piecewise constant and carries no derivative).  So the tangent of the
    state after step 0 is
        J[i, c] = W_b[i, c] + sum over j with idx_0[j] = i of
                  D_0[j] (1 - D_0[j]) h0[j] W_d[j, c],
    later steps carry it forward with the same transitions, V_t = A_t V_{t-1},
    and dy_t / du_0 = C V_t.  Dense, forward-mode, fp64.

    k_star [B,H,L]; dict_idx [H,K,N]; D [B,H,L,N]; W_d, W_b [H,N,d]; C [H,N];
    h0 [B,H,N] or None (zeros).  Returns fp64 [B,H,L,d]."""
    k_star = np.asarray(k_star)
    dict_idx = np.asarray(dict_idx)
    D = np.asarray(D, dtype=F64)
    W_d = np.asarray(W_d, dtype=F64)
    W_b = np.asarray(W_b, dtype=F64)
    C = np.asarray(C, dtype=F64)
    B, H, L = k_star.shape
    N, d = W_d.shape[1], W_d.shape[2]
    h0 = np.zeros((B, H, N), dtype=F64) if h0 is None else np.asarray(h0, dtype=F64)
    out = np.zeros((B, H, L, d), dtype=F64)
    for b in range(B):
        for h in range(H):
            idx0 = dict_idx[h, k_star[b, h, 0]]
            coef = D[b, h, 0] * (1.0 - D[b, h, 0]) * h0[b, h]          # [N]
            V = W_b[h] + transition_matrix(idx0, coef) @ W_d[h]          # [N, d]
            out[b, h, 0] = C[h] @ V
            for t in range(1, L):
                V = transition_matrix(dict_idx[h, k_star[b, h, t]], D[b, h, t]) @ V
                out[b, h, t] = C[h] @ V
    return out


def forward(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0=None, u_shared=False):
    """Selection followed by the sequential scan.

    Returns dict(k_star, D, scores, y, h_L)."""
    k_star, D, s = select(u, W_sel, W_d, b_d, u_shared)
    y, hL = scan(k_star, dict_idx, D, Bu, C, h0)
    return {"k_star": k_star, "D": D, "scores": s, "y": y, "h_L": hL}


def drive(u, W_b, u_shared=False):
    """Drive terms of the recurrence, Bu_t = W_b u_t for every head, in fp64:
    out[b,h,t,n] = sum_c W_b[h,n,c] u[b,(h),t,c] (the input map B of the
    linear SSM in the problem statement of the same summary).  It is the same
    linear form as the scores, with W_b's rows as the outputs."""
    return scores(u, W_b, u_shared)


def forward_wb(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0=None, u_shared=False):
    """``forward`` with the drive terms formed from u and W_b instead of given.

    Returns dict(k_star, D, scores, Bu, y, h_L)."""
    Bu = drive(u, W_b, u_shared)
    out = forward(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0, u_shared)
    out["Bu"] = Bu
    return out


def scan_multi(k_star, dict_idx, D, Bu, C, h0=None):
    """``scan`` with several outputs per head ("Flash PD-SSM" summary,
    methodology item 1, y_t = C h_t with C holding n_out rows per head):
    C [H,n_out,N] gives y[b,h,t,o] = sum_n C[h,o,n] h_t[n], fp64 [B,H,L,n_out];
    returns (y, h_L) with h_L the state after the last step."""
    states = scan_states(k_star, dict_idx, D, Bu, h0)
    C = np.asarray(C, dtype=F64)
    y = np.einsum("bhln,hon->bhlo", states, C)
    return y, states[:, :, -1].copy()


def forward_wb_multi(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0=None, u_shared=False):
    """``forward_wb`` with C [H,n_out,N]: selections, the drive W_b u, then
    ``scan_multi``.  Returns dict(k_star, D, Bu, y [B,H,L,n_out], h_L)."""
    k_star, D, _ = select(u, W_sel, W_d, b_d, u_shared)
    Bu = drive(u, W_b, u_shared)
    y, h_L = scan_multi(k_star, dict_idx, D, Bu, C, h0)
    return {"k_star": k_star, "D": D, "Bu": Bu, "y": y, "h_L": h_L}


def forward_inputs(inp, L=None):
    """``forward`` on a generated input bundle, optionally on its first L steps."""
    c = inp.cfg
    L = c.L if L is None else L
    u = inp.u[:, :L] if c.u_shared else inp.u[:, :, :L]
    return forward(u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d,
                   inp.Bu[:, :, :L], inp.C, inp.h0, c.u_shared)


# --------------------------------------------------------------------------
# PD-map algebra (stated for checking, used by nothing above)
# --------------------------------------------------------------------------

def pd_apply(idx, scale, x, b=None):
    """(P D) x + b by scatter-add: out[idx[j]] += scale[j] * x[j]."""
    idx = np.asarray(idx)
    out = np.zeros(np.shape(x), dtype=F64) if b is None else np.array(b, dtype=F64)
    np.add.at(out, idx, np.asarray(scale, dtype=F64) * np.asarray(x, dtype=F64))
    return out


def pd_compose(later, earlier):
    """Composition later o earlier of two maps (idx, scale): the product of
    their dense matrices, later @ earlier, is again column-one-hot times a
    diagonal, with idx = idx_later[idx_earlier] and
    scale = scale_later[idx_earlier] * scale_earlier."""
    i2, s2 = np.asarray(later[0]), np.asarray(later[1], dtype=F64)
    i1, s1 = np.asarray(earlier[0]), np.asarray(earlier[1], dtype=F64)
    return i2[i1], s2[i1] * s1


# --------------------------------------------------------------------------
# chunked evaluation (phases A, B, C) with dense matrices
# --------------------------------------------------------------------------

def three_phase(k_star, dict_idx, D, Bu, C, h0=None, chunk=64):
    """Chunked evaluation in the pages' three phases, fp64, dense.

    Phase A: each chunk, on its own and from a zero state, runs its steps in
    order, recording local states and the running product of its
    transitions.  Phase B: carries H_c = Phi_c H_{c-1} + b_c from H_{-1} = h0.
    Phase C: h_t = hloc_t + Phi_{c,t} H_{c-1}, y_t = C h_t.
    Returns (y, h_L) like ``scan``."""
    k_star = np.asarray(k_star)
    D = np.asarray(D, dtype=F64)
    Bu = np.asarray(Bu, dtype=F64)
    C = np.asarray(C, dtype=F64)
    B, H, L = k_star.shape
    N = dict_idx.shape[-1]
    starts = list(range(0, L, chunk))
    hloc = np.zeros((B, H, L, N))
    prefix = np.zeros((B, H, L, N, N))          # Phi_{c,t} = A_t ... A_{c0}
    for c0 in starts:                            # phase A (chunks independent)
        x = np.zeros((B, H, N))
        P = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
        for t in range(c0, min(c0 + chunk, L)):
            A = transition_matrix(np.asarray(dict_idx)[np.arange(H)[None, :], k_star[:, :, t]],
                                  D[:, :, t])
            x = np.matmul(A, x[..., None])[..., 0] + Bu[:, :, t]
            P = np.matmul(A, P)
            hloc[:, :, t] = x
            prefix[:, :, t] = P
    carry = np.zeros((B, H, N)) if h0 is None else np.array(h0, dtype=F64)
    carries = []
    for c0 in starts:                            # phase B
        carries.append(carry)
        e = min(c0 + chunk, L) - 1
        carry = np.matmul(prefix[:, :, e], carry[..., None])[..., 0] + hloc[:, :, e]
    y = np.zeros((B, H, L))
    for c0, Hc in zip(starts, carries):          # phase C
        for t in range(c0, min(c0 + chunk, L)):
            h = hloc[:, :, t] + np.matmul(prefix[:, :, t], Hc[..., None])[..., 0]
            y[:, :, t] = (C[None] * h).sum(-1)
    return y, carry

"""Python binding of libpdscan (hard-selection PD-SSM forward pass, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libpdscan.so``, reached through its C ABI (``include/pdscan.h``).
PyTorch supplies device memory and the stream.  Importing this package fails
loudly when the library has not been built; there is no other code path.

Entry points (same names as the C ABI):

* ``pdssm_select(u, W_sel, W_d, b_d, dict_idx=None, want_P=False)``
    -> (k_star, D[, P_idx])
* ``pdssm_scan_fwd(k_star, dict_idx, D, Bu, C, h0=None, chunk=...)``
    -> (y, h_L)
* ``pdssm_fwd(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0=None, chunk=...,
              want_k=False, want_D=False)``
    -> dict(y, h_L[, k_star][, D])

Shapes: u [B,H,L,d] (per head) or [B,L,d] (shared by all heads, detected by
its rank); W_sel [H,K,d]; W_d [H,N,d]; b_d [H,N]; dict_idx [H,K,N] int32;
Bu [B,H,L,N]; C [H,N]; h0 [B,H,N].  u, W_sel and W_d are float32 or bfloat16
(all three the same); everything else float32 / int32.
"""

import ctypes

from ._lib import (  # noqa: F401
    LIB_PATH,
    PDSSM_BF16,
    PDSSM_EHIP,
    PDSSM_EINVAL,
    PDSSM_EUNSUPPORTED,
    PDSSM_EWORKSPACE,
    PDSSM_F32,
    PDSSM_OK,
    PdssmDims,
    PdssmError,
    lib,
)

__all__ = [
    "pdssm_select", "pdssm_scan_fwd", "pdssm_fwd", "pdssm_fwd_wb", "pdssm_impulse_sens",
    "pdssm_soft_select", "pdssm_scan_fwd_pidx", "pdssm_dict_hardmax",
    "pdssm_fwd_wb_multi", "pdssm_scan_fwd_multi",
    "scan_workspace_bytes",
    "fwd_workspace_bytes", "make_dims", "PdssmError", "lib", "LIB_PATH",
]


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _check(rc):
    if rc != PDSSM_OK:
        raise PdssmError(rc, lib.pdssm_last_error().decode())


def make_dims(B, H, L, N, K, d, u_shared=False, bf16=False):
    return PdssmDims(B, H, L, N, K, d, int(bool(u_shared)), PDSSM_BF16 if bf16 else PDSSM_F32)


def _dims_from(u, W_sel, W_d, L=None, B=None):
    torch = _torch()
    if u.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    if W_sel.dtype != u.dtype or W_d.dtype != u.dtype:
        raise TypeError("u, W_sel and W_d must share one dtype")
    H, K, d = W_sel.shape
    N = W_d.shape[1]
    if u.dim() == 4:
        Bv, Hu, Lv, du = u.shape
        shared = False
        if Hu != H:
            raise ValueError("u head count differs from W_sel")
    elif u.dim() == 3:
        Bv, Lv, du = u.shape
        shared = True
    else:
        raise ValueError("u must be [B,H,L,d] or [B,L,d]")
    if du != d or W_d.shape != (H, N, d):
        raise ValueError("inconsistent d / N across u, W_sel, W_d")
    return make_dims(Bv, H, Lv, N, K, d, shared, u.dtype == torch.bfloat16)


def scan_workspace_bytes(dims, chunk):
    n = ctypes.c_size_t(0)
    _check(lib.pdssm_scan_workspace_bytes(ctypes.byref(dims), int(chunk), ctypes.byref(n)))
    return n.value


def fwd_workspace_bytes(dims, chunk):
    n = ctypes.c_size_t(0)
    _check(lib.pdssm_fwd_workspace_bytes(ctypes.byref(dims), int(chunk), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        _need(workspace, "workspace")
        return workspace
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def pdssm_select(u, W_sel, W_d, b_d, dict_idx=None, want_P=False, out=None):
    """Scores, argmax and logistic diagonal on the GPU.  Returns
    (k_star int32 [B,H,L], D float32 [B,H,L,N]) or, with ``want_P``, also the
    selected row-index arrays P_idx int32 [B,H,L,N] (needs dict_idx)."""
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d")):
        _need(t, n)
    _need(b_d, "b_d", torch.float32)
    if dict_idx is not None:
        _need(dict_idx, "dict_idx", torch.int32)
    dims = _dims_from(u, W_sel, W_d)
    dev = u.device
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    o = out or {}
    k = o.get("k_star")
    k = torch.empty((B, H, L), dtype=torch.int32, device=dev) if k is None else _need(k, "k_star")
    D = o.get("D")
    D = torch.empty((B, H, L, N), dtype=torch.float32, device=dev) if D is None else _need(D, "D")
    P = None
    if want_P:
        P = o.get("P_idx")
        P = torch.empty((B, H, L, N), dtype=torch.int32, device=dev) if P is None else _need(P, "P_idx")
    _check(lib.pdssm_select(ctypes.byref(dims), _ptr(u), _ptr(W_sel), _ptr(dict_idx), _ptr(W_d),
                            _ptr(b_d), _ptr(k), _ptr(D), _ptr(P), _stream(dev)))
    return (k, D, P) if want_P else (k, D)


def pdssm_scan_fwd(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """Chunked scan given selections.  Returns (y [B,H,L], h_L [B,H,N])."""
    torch = _torch()
    _need(k_star, "k_star", torch.int32)
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((D, "D"), (Bu, "Bu"), (C, "C")):
        _need(t, n, torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    B, H, L = k_star.shape
    _, K, N = dict_idx.shape
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    y = o.get("y")
    y = torch.empty((B, H, L), dtype=torch.float32, device=dev) if y is None else _need(y, "y")
    hL = o.get("h_L")
    hL = torch.empty((B, H, N), dtype=torch.float32, device=dev) if hL is None else _need(hL, "h_L")
    _check(lib.pdssm_scan_fwd(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                              _ptr(Bu), _ptr(C), _ptr(h0), _ptr(y), _ptr(hL), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev)))
    return y, hL


def pdssm_fwd(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0=None, chunk=128, want_k=False,
              want_D=False, workspace=None, out=None):
    """Fused selection + chunked scan.  Returns dict(y, h_L[, k_star][, D])."""
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d")):
        _need(t, n)
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((b_d, "b_d"), (Bu, "Bu"), (C, "C")):
        _need(t, n, torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    dims = _dims_from(u, W_sel, W_d)
    dev = u.device
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    res = {}
    for name, shape, dt, want in (("y", (B, H, L), torch.float32, True),
                                  ("h_L", (B, H, N), torch.float32, True),
                                  ("k_star", (B, H, L), torch.int32, want_k),
                                  ("D", (B, H, L, N), torch.float32, want_D)):
        if want:
            t = o.get(name)
            res[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_fwd(ctypes.byref(dims), int(chunk), _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                         _ptr(W_d), _ptr(b_d), _ptr(Bu), _ptr(C), _ptr(h0),
                         _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                         _ptr(res["h_L"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


def pdssm_fwd_wb(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0=None, chunk=128, want_k=False,
                 want_D=False, workspace=None, out=None):
    """Fused selection + chunked scan with the drive term Bu = W_b u formed in
    the same pass (W_b [H,N,d] in u's dtype).  Returns dict(y, h_L[, k_star][, D])."""
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d"), (W_b, "W_b")):
        _need(t, n)
    if W_b.dtype != W_d.dtype or tuple(W_b.shape) != tuple(W_d.shape):
        raise ValueError("W_b must have W_d's shape [H,N,d] and dtype")
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((b_d, "b_d"), (C, "C")):
        _need(t, n, torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    dims = _dims_from(u, W_sel, W_d)
    dev = u.device
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    res = {}
    for name, shape, dt, want in (("y", (B, H, L), torch.float32, True),
                                  ("h_L", (B, H, N), torch.float32, True),
                                  ("k_star", (B, H, L), torch.int32, want_k),
                                  ("D", (B, H, L, N), torch.float32, want_D)):
        if want:
            t = o.get(name)
            res[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_fwd_wb(ctypes.byref(dims), int(chunk), _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                            _ptr(W_d), _ptr(b_d), _ptr(W_b), _ptr(C), _ptr(h0),
                            _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                            _ptr(res["h_L"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


def pdssm_fwd_wb_multi(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0=None, chunk=128, want_k=False,
                       want_D=False, workspace=None, out=None):
    """pdssm_fwd_wb with several outputs per head: C [H,n_out,N] (n_out <= 4)
    gives y [B,H,L,n_out].  Returns dict(y, h_L[, k_star][, D])."""
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d"), (W_b, "W_b")):
        _need(t, n)
    if W_b.dtype != W_d.dtype or tuple(W_b.shape) != tuple(W_d.shape):
        raise ValueError("W_b must have W_d's shape [H,N,d] and dtype")
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((b_d, "b_d"), (C, "C")):
        _need(t, n, torch.float32)
    if C.dim() != 3:
        raise ValueError("C must be [H, n_out, N]")
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    dims = _dims_from(u, W_sel, W_d)
    dev = u.device
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    P = int(C.shape[1])
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    res = {}
    for name, shape, dt, want in (("y", (B, H, L, P), torch.float32, True),
                                  ("h_L", (B, H, N), torch.float32, True),
                                  ("k_star", (B, H, L), torch.int32, want_k),
                                  ("D", (B, H, L, N), torch.float32, want_D)):
        if want:
            t = o.get(name)
            res[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_fwd_wb_multi(ctypes.byref(dims), int(chunk), P, _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                                  _ptr(W_d), _ptr(b_d), _ptr(W_b), _ptr(C), _ptr(h0),
                                  _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                                  _ptr(res["h_L"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


def pdssm_scan_fwd_multi(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """pdssm_scan_fwd with several outputs per head: C [H,n_out,N] (n_out <= 4).
    Returns (y [B,H,L,n_out], h_L [B,H,N])."""
    torch = _torch()
    _need(k_star, "k_star", torch.int32)
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((D, "D"), (Bu, "Bu"), (C, "C")):
        _need(t, n, torch.float32)
    if C.dim() != 3:
        raise ValueError("C must be [H, n_out, N]")
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    B, H, L = k_star.shape
    _, K, N = dict_idx.shape
    P = int(C.shape[1])
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    y = o.get("y")
    y = torch.empty((B, H, L, P), dtype=torch.float32, device=dev) if y is None else _need(y, "y")
    hL = o.get("h_L")
    hL = torch.empty((B, H, N), dtype=torch.float32, device=dev) if hL is None else _need(hL, "h_L")
    _check(lib.pdssm_scan_fwd_multi(ctypes.byref(dims), int(chunk), P, _ptr(k_star), _ptr(dict_idx), _ptr(D),
                                    _ptr(Bu), _ptr(C), _ptr(h0), _ptr(y), _ptr(hL), _ptr(ws),
                                    ctypes.c_size_t(ws.numel()), _stream(dev)))
    return y, hL


def impulse_sens_workspace_bytes(dims, chunk):
    n = ctypes.c_size_t(0)
    _check(lib.pdssm_impulse_sens_workspace_bytes(ctypes.byref(dims), int(chunk), ctypes.byref(n)))
    return n.value


def pdssm_impulse_sens(k_star, dict_idx, D, W_d, W_b, C, h0=None, chunk=128, workspace=None, out=None):
    """dy_t / du_0 for fixed selections: returns dY [B,H,L,d] fp32.  W_d and W_b
    [H,N,d] share a dtype (fp32 or bf16)."""
    torch = _torch()
    _need(k_star, "k_star", torch.int32)
    _need(dict_idx, "dict_idx", torch.int32)
    _need(D, "D", torch.float32)
    _need(C, "C", torch.float32)
    _need(W_d, "W_d")
    _need(W_b, "W_b")
    if W_b.dtype != W_d.dtype or tuple(W_b.shape) != tuple(W_d.shape):
        raise ValueError("W_b must have W_d's shape [H,N,d] and dtype")
    if W_d.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("W_d and W_b must be float32 or bfloat16")
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    B, H, L = k_star.shape
    K, N = dict_idx.shape[1], dict_idx.shape[2]
    d = W_d.shape[2]
    dims = make_dims(B, H, L, N, K, d, 0, W_d.dtype == torch.bfloat16)
    dev = k_star.device
    ws = _workspace(impulse_sens_workspace_bytes(dims, chunk), dev, workspace)
    dY = torch.empty((B, H, L, d), dtype=torch.float32, device=dev) if out is None else _need(out, "dY")
    _check(lib.pdssm_impulse_sens(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                                  _ptr(W_d), _ptr(W_b), _ptr(C), _ptr(h0), _ptr(dY), _ptr(ws),
                                  ctypes.c_size_t(ws.numel()), _stream(dev)))
    return dY


def pdssm_soft_select(u, W_sel, M, W_d, b_d, out=None):
    """Soft-selection comparison path: returns dict(M_t, P_idx, D).  M is
    [H,K,N,N] fp32 (row i, column j)."""
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d")):
        _need(t, n)
    for t, n in ((M, "M"), (b_d, "b_d")):
        _need(t, n, torch.float32)
    dims = _dims_from(u, W_sel, W_d)
    dev = u.device
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    o = out or {}
    res = {}
    for name, shape, dt in (("M_t", (B, H, L, N, N), torch.float32), ("P_idx", (B, H, L, N), torch.int32),
                            ("D", (B, H, L, N), torch.float32)):
        t = o.get(name)
        res[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_soft_select(ctypes.byref(dims), _ptr(u), _ptr(W_sel), _ptr(M), _ptr(W_d), _ptr(b_d),
                                 _ptr(res["M_t"]), _ptr(res["P_idx"]), _ptr(res["D"]), _stream(dev)))
    return res


def pdssm_scan_fwd_pidx(P_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """The scan on per-step column maps P_idx [B,H,L,N].  Returns (y, h_L)."""
    torch = _torch()
    _need(P_idx, "P_idx", torch.int32)
    for t, n in ((D, "D"), (Bu, "Bu"), (C, "C")):
        _need(t, n, torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    B, H, L, N = P_idx.shape
    dims = make_dims(B, H, L, N, 1, 8, 0, False)
    dev = P_idx.device
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    y = o.get("y")
    y = torch.empty((B, H, L), dtype=torch.float32, device=dev) if y is None else _need(y, "y")
    hL = o.get("h_L")
    hL = torch.empty((B, H, N), dtype=torch.float32, device=dev) if hL is None else _need(hL, "h_L")
    _check(lib.pdssm_scan_fwd_pidx(ctypes.byref(dims), int(chunk), _ptr(P_idx), _ptr(D), _ptr(Bu), _ptr(C),
                                   _ptr(h0), _ptr(y), _ptr(hL), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                   _stream(dev)))
    return y, hL


def pdssm_dict_hardmax(M):
    """dict_idx[h,k,j] = lowest row i with M[h,k,i,j] maximal; M [H,K,N,N] fp32."""
    torch = _torch()
    _need(M, "M", torch.float32)
    H, K, N, N2 = M.shape
    if N != N2:
        raise ValueError("M must be [H,K,N,N]")
    out = torch.empty((H, K, N), dtype=torch.int32, device=M.device)
    _check(lib.pdssm_dict_hardmax(int(H), int(K), int(N), _ptr(M), _ptr(out), _stream(M.device)))
    return out


def scan_bwd_workspace_bytes(dims, chunk):
    n = ctypes.c_size_t(0)
    _check(lib.pdssm_scan_bwd_workspace_bytes(ctypes.byref(dims), int(chunk), ctypes.byref(n)))
    return n.value


def _scan_dims(k_star, dict_idx):
    B, H, L = k_star.shape
    _, K, N = dict_idx.shape
    return make_dims(B, H, L, N, K, 8)


def pdssm_scan_states(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """Chunked scan that also returns the state after every step.  Returns
    (y [B,H,L], h_L [B,H,N], H_all [B,H,L,N])."""
    torch = _torch()
    _need(k_star, "k_star", torch.int32)
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((D, "D"), (Bu, "Bu"), (C, "C")):
        _need(t, n, torch.float32)
    if h0 is not None:
        _need(h0, "h0", torch.float32)
    dims = _scan_dims(k_star, dict_idx)
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    dev = k_star.device
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    res = {}
    for name, shape in (("y", (B, H, L)), ("h_L", (B, H, N)), ("H_all", (B, H, L, N))):
        t = o.get(name)
        res[name] = torch.empty(shape, dtype=torch.float32, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_scan_states(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                                 _ptr(Bu), _ptr(C), _ptr(h0), _ptr(res["y"]), _ptr(res["h_L"]),
                                 _ptr(res["H_all"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res["y"], res["h_L"], res["H_all"]


def pdssm_scan_bwd(k_star, dict_idx, D, C, H_all, g_y, h0=None, g_hL=None, chunk=128,
                   want_h0=True, workspace=None, out=None):
    """Gradient through the scan for fixed selections.  Returns
    dict(g_Bu [B,H,L,N], g_D [B,H,L,N], g_C [H,N][, g_h0 [B,H,N]])."""
    torch = _torch()
    _need(k_star, "k_star", torch.int32)
    _need(dict_idx, "dict_idx", torch.int32)
    for t, n in ((D, "D"), (C, "C"), (H_all, "H_all"), (g_y, "g_y")):
        _need(t, n, torch.float32)
    for t, n in ((h0, "h0"), (g_hL, "g_hL")):
        if t is not None:
            _need(t, n, torch.float32)
    dims = _scan_dims(k_star, dict_idx)
    B, H, L, N = dims.B, dims.H, dims.L, dims.N
    dev = k_star.device
    ws = _workspace(scan_bwd_workspace_bytes(dims, chunk), dev, workspace)
    o = out or {}
    res = {}
    for name, shape, want in (("g_Bu", (B, H, L, N), True), ("g_D", (B, H, L, N), True),
                              ("g_h0", (B, H, N), want_h0), ("g_C", (H, N), True)):
        if want:
            t = o.get(name)
            res[name] = torch.empty(shape, dtype=torch.float32, device=dev) if t is None else _need(t, name)
    _check(lib.pdssm_scan_bwd(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                              _ptr(C), _ptr(h0), _ptr(H_all), _ptr(g_y), _ptr(g_hL), _ptr(res["g_Bu"]),
                              _ptr(res["g_D"]), _ptr(res.get("g_h0")), _ptr(res["g_C"]), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


__all__ += ["scan_bwd_workspace_bytes", "pdssm_scan_states", "pdssm_scan_bwd"]


def workspace_error_flag(workspace):
    """Nonzero if a look-back wait in the last call on ``workspace`` gave up
    (read after synchronising).  Header word 1 of the workspace."""
    return int(workspace[4:8].view(_torch().int32).item())


__all__.append("workspace_error_flag")

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
    PDSSM_NOALLOC_SCRATCH_BYTES,
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
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _args(*specs):
    """Check tensor arguments against the call's dims before anything reaches
    the library: the C ABI cannot see allocation sizes, so a tensor of the
    wrong shape or dtype would be read or written past its end on the device.
    Each spec is (tensor or None, name, shape, dtype); None tensors are
    optional arguments left out.  Types, dtypes and shapes of every argument
    are checked first, then device placement and contiguity."""
    torch = _torch()
    present = [sp for sp in specs if sp[0] is not None]
    for t, name, shape, dtype in present:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
        if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)} (got {tuple(t.shape)})")
    for t, name, _, _ in present:
        _need(t, name)


def _out(o, name, shape, dtype, dev):
    """A caller-supplied output (checked by _args afterwards) or a new one."""
    t = o.get(name)
    if t is None:
        return _torch().empty(tuple(shape), dtype=dtype, device=dev)
    return t


def _check(rc):
    if rc != PDSSM_OK:
        raise PdssmError(rc, lib.pdssm_last_error().decode())


def make_dims(B, H, L, N, K, d, u_shared=False, bf16=False):
    return PdssmDims(B, H, L, N, K, d, int(bool(u_shared)), PDSSM_BF16 if bf16 else PDSSM_F32)


def _dims_from(u, W_sel, W_d, L=None, B=None):
    torch = _torch()
    for t, n in ((u, "u"), (W_sel, "W_sel"), (W_d, "W_d")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
    if u.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    if W_sel.dtype != u.dtype or W_d.dtype != u.dtype:
        raise TypeError("u, W_sel and W_d must share one dtype")
    if W_sel.dim() != 3 or W_d.dim() != 3:
        raise ValueError("W_sel must be [H,K,d] and W_d [H,N,d]")
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
        _need(workspace, "workspace", torch.uint8)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")
        return workspace
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _scan_shape(k_star, dict_idx):
    """B, H, L from k_star [B,H,L]; K, N from dict_idx [H,K,N]."""
    torch = _torch()
    for t, n in ((k_star, "k_star"), (dict_idx, "dict_idx")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.dim() != 3:
            raise ValueError(f"{n} must have three dimensions")
    B, H, L = k_star.shape
    if dict_idx.shape[0] != H:
        raise ValueError(f"dict_idx has {dict_idx.shape[0]} heads, k_star {H}")
    return B, H, L, dict_idx.shape[1], dict_idx.shape[2]


def _fwd_common(u, W_sel, W_d):
    dims = _dims_from(u, W_sel, W_d)
    return dims, dims.B, dims.H, dims.L, dims.N, dims.K, dims.d_in


def pdssm_select(u, W_sel, W_d, b_d, dict_idx=None, want_P=False, out=None):
    """Scores, argmax and logistic diagonal on the GPU.  Returns
    (k_star int32 [B,H,L], D float32 [B,H,L,N]) or, with ``want_P``, also the
    selected row-index arrays P_idx int32 [B,H,L,N] (needs dict_idx)."""
    torch = _torch()
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    dev = u.device
    o = out or {}
    k = _out(o, "k_star", (B, H, L), torch.int32, dev)
    D = _out(o, "D", (B, H, L, N), torch.float32, dev)
    P = _out(o, "P_idx", (B, H, L, N), torch.int32, dev) if want_P else None
    _args((u, "u", None, None), (W_sel, "W_sel", None, None), (W_d, "W_d", None, None),
          (b_d, "b_d", (H, N), torch.float32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (k, "k_star", (B, H, L), torch.int32), (D, "D", (B, H, L, N), torch.float32),
          (P, "P_idx", (B, H, L, N), torch.int32))
    _check(lib.pdssm_select(ctypes.byref(dims), _ptr(u), _ptr(W_sel), _ptr(dict_idx), _ptr(W_d),
                            _ptr(b_d), _ptr(k), _ptr(D), _ptr(P), _stream(dev)))
    return (k, D, P) if want_P else (k, D)


def pdssm_scan_fwd(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """Chunked scan given selections.  Returns (y [B,H,L], h_L [B,H,N])."""
    torch = _torch()
    B, H, L, K, N = _scan_shape(k_star, dict_idx)
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    o = out or {}
    y = _out(o, "y", (B, H, L), torch.float32, dev)
    hL = _out(o, "h_L", (B, H, N), torch.float32, dev)
    _args((k_star, "k_star", (B, H, L), torch.int32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (D, "D", (B, H, L, N), torch.float32), (Bu, "Bu", (B, H, L, N), torch.float32),
          (C, "C", (H, N), torch.float32), (h0, "h0", (B, H, N), torch.float32),
          (y, "y", (B, H, L), torch.float32), (hL, "h_L", (B, H, N), torch.float32))
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_scan_fwd(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                              _ptr(Bu), _ptr(C), _ptr(h0), _ptr(y), _ptr(hL), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev)))
    return y, hL


def _fwd_outputs(o, B, H, L, N, want_k, want_D, dev, n_out=None):
    torch = _torch()
    res = {"y": _out(o, "y", (B, H, L) if n_out is None else (B, H, L, n_out), torch.float32, dev),
           "h_L": _out(o, "h_L", (B, H, N), torch.float32, dev)}
    if want_k:
        res["k_star"] = _out(o, "k_star", (B, H, L), torch.int32, dev)
    if want_D:
        res["D"] = _out(o, "D", (B, H, L, N), torch.float32, dev)
    return res


def _fwd_out_specs(res, B, H, L, N, n_out=None):
    torch = _torch()
    return ((res["y"], "y", (B, H, L) if n_out is None else (B, H, L, n_out), torch.float32),
            (res["h_L"], "h_L", (B, H, N), torch.float32),
            (res.get("k_star"), "k_star", (B, H, L), torch.int32),
            (res.get("D"), "D", (B, H, L, N), torch.float32))


def pdssm_fwd(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0=None, chunk=128, want_k=False,
              want_D=False, workspace=None, out=None):
    """Fused selection + chunked scan.  Returns dict(y, h_L[, k_star][, D])."""
    torch = _torch()
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    dev = u.device
    res = _fwd_outputs(out or {}, B, H, L, N, want_k, want_D, dev)
    _args((u, "u", None, None), (W_sel, "W_sel", None, None), (W_d, "W_d", None, None),
          (dict_idx, "dict_idx", (H, K, N), torch.int32), (b_d, "b_d", (H, N), torch.float32),
          (Bu, "Bu", (B, H, L, N), torch.float32), (C, "C", (H, N), torch.float32),
          (h0, "h0", (B, H, N), torch.float32), *_fwd_out_specs(res, B, H, L, N))
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_fwd(ctypes.byref(dims), int(chunk), _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                         _ptr(W_d), _ptr(b_d), _ptr(Bu), _ptr(C), _ptr(h0),
                         _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                         _ptr(res["h_L"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


def pdssm_fwd_noalloc(u, W_sel, dict_idx, W_d, b_d, Bu, C, h0=None, chunk=128, want_k=False,
                      want_D=False, status=None, out=None):
    """pdssm_fwd without a workspace: the look-back scratch is the library's
    own per-device array (calls on one GPU must not overlap).  ``status`` (a
    device int32 tensor of one element, optional) receives the look-back
    error word ORed in.  Returns dict(y, h_L[, k_star][, D])."""
    torch = _torch()
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    dev = u.device
    res = _fwd_outputs(out or {}, B, H, L, N, want_k, want_D, dev)
    _args((u, "u", None, None), (W_sel, "W_sel", None, None), (W_d, "W_d", None, None),
          (dict_idx, "dict_idx", (H, K, N), torch.int32), (b_d, "b_d", (H, N), torch.float32),
          (Bu, "Bu", (B, H, L, N), torch.float32), (C, "C", (H, N), torch.float32),
          (h0, "h0", (B, H, N), torch.float32), (status, "status", (1,), torch.int32),
          *_fwd_out_specs(res, B, H, L, N))
    _check(lib.pdssm_fwd_noalloc(ctypes.byref(dims), int(chunk), _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                                 _ptr(W_d), _ptr(b_d), _ptr(Bu), _ptr(C), _ptr(h0),
                                 _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                                 _ptr(res["h_L"]), _ptr(status), _stream(dev)))
    return res


def _wb_args(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0, res, B, H, L, N, K, d, n_out=None):
    torch = _torch()
    _args((u, "u", None, None), (W_sel, "W_sel", None, None), (W_d, "W_d", None, None),
          (W_b, "W_b", (H, N, d), W_d.dtype), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (b_d, "b_d", (H, N), torch.float32),
          (C, "C", (H, N) if n_out is None else (H, n_out, N), torch.float32),
          (h0, "h0", (B, H, N), torch.float32), *_fwd_out_specs(res, B, H, L, N, n_out))


def pdssm_fwd_wb(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0=None, chunk=128, want_k=False,
                 want_D=False, workspace=None, out=None):
    """Fused selection + chunked scan with the drive term Bu = W_b u formed in
    the same pass (W_b [H,N,d] in u's dtype).  Returns dict(y, h_L[, k_star][, D])."""
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    dev = u.device
    res = _fwd_outputs(out or {}, B, H, L, N, want_k, want_D, dev)
    _wb_args(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0, res, B, H, L, N, K, d)
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
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
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    if not isinstance(C, torch.Tensor) or C.dim() != 3:
        raise ValueError("C must be [H, n_out, N]")
    P = int(C.shape[1])
    dev = u.device
    res = _fwd_outputs(out or {}, B, H, L, N, want_k, want_D, dev, n_out=P)
    _wb_args(u, W_sel, dict_idx, W_d, b_d, W_b, C, h0, res, B, H, L, N, K, d, n_out=P)
    ws = _workspace(fwd_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_fwd_wb_multi(ctypes.byref(dims), int(chunk), P, _ptr(u), _ptr(W_sel), _ptr(dict_idx),
                                  _ptr(W_d), _ptr(b_d), _ptr(W_b), _ptr(C), _ptr(h0),
                                  _ptr(res.get("k_star")), _ptr(res.get("D")), _ptr(res["y"]),
                                  _ptr(res["h_L"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


def pdssm_scan_fwd_multi(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """pdssm_scan_fwd with several outputs per head: C [H,n_out,N] (n_out <= 4).
    Returns (y [B,H,L,n_out], h_L [B,H,N])."""
    torch = _torch()
    B, H, L, K, N = _scan_shape(k_star, dict_idx)
    if not isinstance(C, torch.Tensor) or C.dim() != 3:
        raise ValueError("C must be [H, n_out, N]")
    P = int(C.shape[1])
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    o = out or {}
    y = _out(o, "y", (B, H, L, P), torch.float32, dev)
    hL = _out(o, "h_L", (B, H, N), torch.float32, dev)
    _args((k_star, "k_star", (B, H, L), torch.int32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (D, "D", (B, H, L, N), torch.float32), (Bu, "Bu", (B, H, L, N), torch.float32),
          (C, "C", (H, P, N), torch.float32), (h0, "h0", (B, H, N), torch.float32),
          (y, "y", (B, H, L, P), torch.float32), (hL, "h_L", (B, H, N), torch.float32))
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
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
    B, H, L, K, N = _scan_shape(k_star, dict_idx)
    if not isinstance(W_d, torch.Tensor) or W_d.dim() != 3:
        raise ValueError("W_d must be [H,N,d]")
    if W_d.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W_d and W_b must be float32 or bfloat16")
    d = int(W_d.shape[2])
    dims = make_dims(B, H, L, N, K, d, 0, W_d.dtype == torch.bfloat16)
    dev = k_star.device
    dY = torch.empty((B, H, L, d), dtype=torch.float32, device=dev) if out is None else out
    _args((k_star, "k_star", (B, H, L), torch.int32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (D, "D", (B, H, L, N), torch.float32), (W_d, "W_d", (H, N, d), None),
          (W_b, "W_b", (H, N, d), W_d.dtype), (C, "C", (H, N), torch.float32),
          (h0, "h0", (B, H, N), torch.float32), (dY, "dY", (B, H, L, d), torch.float32))
    ws = _workspace(impulse_sens_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_impulse_sens(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                                  _ptr(W_d), _ptr(W_b), _ptr(C), _ptr(h0), _ptr(dY), _ptr(ws),
                                  ctypes.c_size_t(ws.numel()), _stream(dev)))
    return dY


def pdssm_soft_select(u, W_sel, M, W_d, b_d, out=None):
    """Soft-selection comparison path: returns dict(M_t, P_idx, D).  M is
    [H,K,N,N] fp32 (row i, column j)."""
    torch = _torch()
    dims, B, H, L, N, K, d = _fwd_common(u, W_sel, W_d)
    dev = u.device
    o = out or {}
    res = {"M_t": _out(o, "M_t", (B, H, L, N, N), torch.float32, dev),
           "P_idx": _out(o, "P_idx", (B, H, L, N), torch.int32, dev),
           "D": _out(o, "D", (B, H, L, N), torch.float32, dev)}
    _args((u, "u", None, None), (W_sel, "W_sel", None, None), (W_d, "W_d", None, None),
          (M, "M", (H, K, N, N), torch.float32), (b_d, "b_d", (H, N), torch.float32),
          (res["M_t"], "M_t", (B, H, L, N, N), torch.float32),
          (res["P_idx"], "P_idx", (B, H, L, N), torch.int32), (res["D"], "D", (B, H, L, N), torch.float32))
    _check(lib.pdssm_soft_select(ctypes.byref(dims), _ptr(u), _ptr(W_sel), _ptr(M), _ptr(W_d), _ptr(b_d),
                                 _ptr(res["M_t"]), _ptr(res["P_idx"]), _ptr(res["D"]), _stream(dev)))
    return res


def pdssm_scan_fwd_pidx(P_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """The scan on per-step column maps P_idx [B,H,L,N].  Returns (y, h_L)."""
    torch = _torch()
    if not isinstance(P_idx, torch.Tensor) or P_idx.dim() != 4:
        raise ValueError("P_idx must be [B,H,L,N]")
    B, H, L, N = P_idx.shape
    dims = make_dims(B, H, L, N, 1, 8, 0, False)
    dev = P_idx.device
    o = out or {}
    y = _out(o, "y", (B, H, L), torch.float32, dev)
    hL = _out(o, "h_L", (B, H, N), torch.float32, dev)
    _args((P_idx, "P_idx", (B, H, L, N), torch.int32), (D, "D", (B, H, L, N), torch.float32),
          (Bu, "Bu", (B, H, L, N), torch.float32), (C, "C", (H, N), torch.float32),
          (h0, "h0", (B, H, N), torch.float32), (y, "y", (B, H, L), torch.float32),
          (hL, "h_L", (B, H, N), torch.float32))
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_scan_fwd_pidx(ctypes.byref(dims), int(chunk), _ptr(P_idx), _ptr(D), _ptr(Bu), _ptr(C),
                                   _ptr(h0), _ptr(y), _ptr(hL), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                   _stream(dev)))
    return y, hL


def pdssm_dict_hardmax(M):
    """dict_idx[h,k,j] = lowest row i with M[h,k,i,j] maximal; M [H,K,N,N] fp32."""
    torch = _torch()
    _need(M, "M", torch.float32)
    if M.dim() != 4:
        raise ValueError("M must be [H,K,N,N]")
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


def pdssm_scan_states(k_star, dict_idx, D, Bu, C, h0=None, chunk=128, workspace=None, out=None):
    """Chunked scan that also returns the state after every step.  Returns
    (y [B,H,L], h_L [B,H,N], H_all [B,H,L,N])."""
    torch = _torch()
    B, H, L, K, N = _scan_shape(k_star, dict_idx)
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    o = out or {}
    res = {"y": _out(o, "y", (B, H, L), torch.float32, dev),
           "h_L": _out(o, "h_L", (B, H, N), torch.float32, dev),
           "H_all": _out(o, "H_all", (B, H, L, N), torch.float32, dev)}
    _args((k_star, "k_star", (B, H, L), torch.int32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (D, "D", (B, H, L, N), torch.float32), (Bu, "Bu", (B, H, L, N), torch.float32),
          (C, "C", (H, N), torch.float32), (h0, "h0", (B, H, N), torch.float32),
          (res["y"], "y", (B, H, L), torch.float32), (res["h_L"], "h_L", (B, H, N), torch.float32),
          (res["H_all"], "H_all", (B, H, L, N), torch.float32))
    ws = _workspace(scan_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_scan_states(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                                 _ptr(Bu), _ptr(C), _ptr(h0), _ptr(res["y"]), _ptr(res["h_L"]),
                                 _ptr(res["H_all"]), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res["y"], res["h_L"], res["H_all"]


def pdssm_scan_bwd(k_star, dict_idx, D, C, H_all, g_y, h0=None, g_hL=None, chunk=128,
                   want_h0=True, workspace=None, out=None):
    """Gradient through the scan for fixed selections.  Returns
    dict(g_Bu [B,H,L,N], g_D [B,H,L,N], g_C [H,N][, g_h0 [B,H,N]])."""
    torch = _torch()
    B, H, L, K, N = _scan_shape(k_star, dict_idx)
    dims = make_dims(B, H, L, N, K, 8)
    dev = k_star.device
    o = out or {}
    res = {"g_Bu": _out(o, "g_Bu", (B, H, L, N), torch.float32, dev),
           "g_D": _out(o, "g_D", (B, H, L, N), torch.float32, dev),
           "g_C": _out(o, "g_C", (H, N), torch.float32, dev)}
    if want_h0:
        res["g_h0"] = _out(o, "g_h0", (B, H, N), torch.float32, dev)
    f32 = torch.float32
    _args((k_star, "k_star", (B, H, L), torch.int32), (dict_idx, "dict_idx", (H, K, N), torch.int32),
          (D, "D", (B, H, L, N), f32), (C, "C", (H, N), f32), (H_all, "H_all", (B, H, L, N), f32),
          (g_y, "g_y", (B, H, L), f32), (h0, "h0", (B, H, N), f32), (g_hL, "g_hL", (B, H, N), f32),
          (res["g_Bu"], "g_Bu", (B, H, L, N), f32), (res["g_D"], "g_D", (B, H, L, N), f32),
          (res["g_C"], "g_C", (H, N), f32), (res.get("g_h0"), "g_h0", (B, H, N), f32))
    ws = _workspace(scan_bwd_workspace_bytes(dims, chunk), dev, workspace)
    _check(lib.pdssm_scan_bwd(ctypes.byref(dims), int(chunk), _ptr(k_star), _ptr(dict_idx), _ptr(D),
                              _ptr(C), _ptr(h0), _ptr(H_all), _ptr(g_y), _ptr(g_hL), _ptr(res["g_Bu"]),
                              _ptr(res["g_D"]), _ptr(res.get("g_h0")), _ptr(res["g_C"]), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev)))
    return res


__all__ += ["scan_bwd_workspace_bytes", "pdssm_scan_states", "pdssm_scan_bwd"]


def pdssm_workspace_status(workspace, status=None):
    """Enqueue, on the current stream, status[0] |= the look-back error word of
    the last call on ``workspace`` (nonzero: a wait gave up and that call's
    outputs are wrong).  ``status`` is a device int32 tensor of one element
    (zeroed here when not given); returns it.  Read it after synchronising."""
    torch = _torch()
    _need(workspace, "workspace", torch.uint8)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    _args((status, "status", (1,), torch.int32))
    _check(lib.pdssm_workspace_status(_ptr(workspace), ctypes.c_size_t(workspace.numel()), _ptr(status),
                                      _stream(workspace.device)))
    return status


def workspace_error_flag(workspace):
    """Nonzero if a look-back wait in the last call on ``workspace`` gave up
    (synchronises; the value of pdssm_workspace_status)."""
    st = pdssm_workspace_status(workspace)
    return int(st.item())


__all__ += ["pdssm_workspace_status", "workspace_error_flag", "pdssm_fwd_noalloc"]

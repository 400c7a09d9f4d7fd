"""Helpers shared by the GPU tests: upload generated inputs, call the library
through its binding, compare with the oracle."""

import numpy as np

TOL = 1e-4          # |gpu - ref| <= TOL * (1 + |ref|) for y and h_L


def torch_mod():
    import torch
    return torch


def lib():
    from tests._libutil import ensure_built
    ensure_built()
    import structured_sparse_state_pdssm_amd as P
    return P


def to_dev(x, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def proj_dev(x, bf16):
    """Upload u / W_sel / W_d: fp32 as is, or bf16 (the values are already
    bf16-representable, so the conversion is exact)."""
    torch = torch_mod()
    return to_dev(x, torch.bfloat16 if bf16 else torch.float32)


def upload(inp):
    c = inp.cfg
    bf = c.dtype == "bf16"
    return dict(
        u=proj_dev(inp.u, bf), W_sel=proj_dev(inp.W_sel, bf), W_d=proj_dev(inp.W_d, bf),
        b_d=to_dev(inp.b_d), dict_idx=to_dev(inp.dict_idx), Bu=to_dev(inp.Bu), C=to_dev(inp.C),
        h0=to_dev(inp.h0))


def within(gpu, ref, tol=TOL):
    """Elementwise bound; returns (ok, worst ratio)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ratio = np.abs(gpu - ref) / (tol * (1.0 + np.abs(ref)))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.isfinite(gpu).all() and worst <= 1.0), worst


def assert_within(gpu, ref, what, tol=TOL):
    ok, worst = within(gpu, ref, tol)
    assert ok, f"{what}: worst |err| / ({tol:g}(1+|ref|)) = {worst:.3g}"


def run_fwd(dev, chunk, want=True, h0=True, workspace=None):
    P = lib()
    return P.pdssm_fwd(dev["u"], dev["W_sel"], dev["dict_idx"], dev["W_d"], dev["b_d"], dev["Bu"],
                       dev["C"], dev["h0"] if h0 else None, chunk=chunk, want_k=want, want_D=want,
                       workspace=workspace)


def host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()

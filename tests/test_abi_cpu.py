"""The C ABI library on the host, no GPU: it loads, exports every entry point
that include/pdscan.h declares, and rejects bad arguments before any HIP call
(these calls never reach a kernel launch)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def P():
    from tests._libutil import ensure_built
    ensure_built()
    import structured_sparse_state_pdssm_amd as P
    return P


def _declared():
    with open(os.path.join(ROOT, "include", "pdscan.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:int|const char\*|size_t)\s+(pdssm_\w+)\(", text, re.M)))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("pdssm_select", "pdssm_scan_fwd", "pdssm_fwd", "pdssm_scan_workspace_bytes",
              "pdssm_fwd_workspace_bytes", "pdssm_status_str", "pdssm_last_error",
              "pdssm_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(P):
    lib = ctypes.CDLL(P.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert P.lib.pdssm_abi_version() == 1


def test_status_strings(P):
    for code, text in ((0, b"ok"), (-1, b"invalid argument"), (-2, b"unsupported shape"),
                       (-3, b"workspace too small"), (-4, b"HIP error"), (7, b"unknown status")):
        assert P.lib.pdssm_status_str(code) == text


def _dims(P, **kw):
    base = dict(B=1, H=32, L=131072, N=16, K=8, d=64, u_shared=False, bf16=False)
    base.update(kw)
    return P.make_dims(**base)


def test_workspace_sizes(P):
    d = _dims(P)
    n = P.fwd_workspace_bytes(d, 512)
    # header + (3N aggregate + N inclusive) tagged 8-byte words per chunk and sequence
    assert n == 256 + 256 * 32 * 4 * 16 * 8
    assert P.scan_workspace_bytes(d, 512) == n
    assert P.fwd_workspace_bytes(_dims(P, L=1000), 512) == 256 + 2 * 32 * 4 * 16 * 8


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, -1), ("H", -1, -1), ("L", 0, -1), ("N", 0, -1), ("K", 0, -1), ("d", 0, -1),
    ("N", 65, -2), ("K", 65, -2), ("d", 12, -2), ("d", 8200, -2),
])
def test_bad_dims_rejected(P, field, value, code):
    d = _dims(P, **{field: value})
    n = ctypes.c_size_t(0)
    rc = P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(d), 128, ctypes.byref(n))
    assert rc == code
    assert P.lib.pdssm_last_error() != b""


def test_bad_enums_and_chunk(P):
    n = ctypes.c_size_t(0)
    d = _dims(P)
    d.in_dtype = 7
    assert P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(d), 128, ctypes.byref(n)) == -1
    d = _dims(P)
    d.u_shared = 2
    assert P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(d), 128, ctypes.byref(n)) == -1
    d = _dims(P)
    assert P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(n)) == -1
    assert P.lib.pdssm_fwd_workspace_bytes(None, 16, ctypes.byref(n)) == -1
    assert P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(d), 16, None) == -1
    # a chunk whose on-chip footprint exceeds the limit
    assert P.lib.pdssm_fwd_workspace_bytes(ctypes.byref(_dims(P, N=64)), 512,
                                           ctypes.byref(n)) == -2
    assert b"on-chip" in P.lib.pdssm_last_error()


# Fake, never-dereferenced device addresses: every call below fails validation
# before any HIP call is made.
A = 0x7f0000000000


def _fwd_args(P, **over):
    d = _dims(P, L=2048)
    ws = P.fwd_workspace_bytes(d, 128)
    big = 1 << 30
    args = dict(dims=d, chunk=128, u=A, W_sel=A + big, dict_idx=A + 2 * big, W_d=A + 3 * big,
                b_d=A + 4 * big, Bu=A + 5 * big, C=A + 6 * big, h0=None, k_star=None, D=None,
                y=A + 7 * big, h_L=A + 8 * big, ws=A + 9 * big, ws_bytes=ws, stream=None)
    args.update(over)
    return args


def _call_fwd(P, a):
    return P.lib.pdssm_fwd(ctypes.byref(a["dims"]), a["chunk"], a["u"], a["W_sel"], a["dict_idx"],
                           a["W_d"], a["b_d"], a["Bu"], a["C"], a["h0"], a["k_star"], a["D"],
                           a["y"], a["h_L"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("name", ["u", "W_sel", "dict_idx", "W_d", "b_d", "Bu", "C", "y", "h_L", "ws"])
def test_fwd_null_required(P, name):
    a = _fwd_args(P, **{name: None})
    assert _call_fwd(P, a) == -1
    assert b"NULL" in P.lib.pdssm_last_error()


def test_fwd_misaligned(P):
    a = _fwd_args(P, Bu=A + (5 << 30) + 4)
    assert _call_fwd(P, a) == -1
    assert b"aligned" in P.lib.pdssm_last_error()


def test_fwd_aliasing(P):
    a = _fwd_args(P, y=A + (5 << 30) + 64)          # y inside Bu
    assert _call_fwd(P, a) == -1
    assert b"overlaps" in P.lib.pdssm_last_error()
    a = _fwd_args(P, k_star=A + (8 << 30))           # k_star on top of h_L
    assert _call_fwd(P, a) == -1


def test_fwd_small_workspace(P):
    a = _fwd_args(P)
    a["ws_bytes"] -= 8
    assert _call_fwd(P, a) == -3


def test_select_and_scan_validation(P):
    d = _dims(P, L=2048)
    big = 1 << 30
    # P_idx requested without a dictionary
    rc = P.lib.pdssm_select(ctypes.byref(d), A, A + big, None, A + 2 * big, A + 3 * big,
                            A + 4 * big, A + 5 * big, A + 6 * big, None)
    assert rc == -1 and b"dict_idx" in P.lib.pdssm_last_error()
    # D missing
    rc = P.lib.pdssm_select(ctypes.byref(d), A, A + big, None, A + 2 * big, A + 3 * big,
                            A + 4 * big, None, None, None)
    assert rc == -1
    ws = P.scan_workspace_bytes(d, 64)
    rc = P.lib.pdssm_scan_fwd(ctypes.byref(d), 64, A, A + big, A + 2 * big, A + 3 * big,
                              A + 4 * big, None, A + 5 * big, A + 6 * big, A + 7 * big, ws - 1, None)
    assert rc == -3
    rc = P.lib.pdssm_scan_fwd(ctypes.byref(d), 64, A, None, A + 2 * big, A + 3 * big,
                              A + 4 * big, None, A + 5 * big, A + 6 * big, A + 7 * big, ws, None)
    assert rc == -1


def test_binding_rejects_host_tensors(P):
    import torch
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        P.pdssm_scan_fwd(torch.zeros((1, 1, 4), dtype=torch.int32), torch.zeros((1, 1, 2), dtype=torch.int32),
                         x, x, x)


def test_multi_output_validation(P):
    """n_out outside [1, 4]: invalid; a chunk whose per-output on-chip rows do
    not fit, or a shape off the step-major paths: unsupported; a fitting call
    then fails only on its (empty) workspace."""
    big = 1 << 30
    d = _dims(P, L=4096)
    args = lambda ws: (A, A + big, A + 2 * big, A + 3 * big, A + 4 * big, None,  # noqa: E731
                       A + 5 * big, A + 6 * big, A + 7 * big, ws, None)
    for n_out, chunk, want in ((0, 128, -1), (5, 128, -1), (2, 512, -2), (4, 256, -2), (4, 128, -3),
                               (2, 256, -3)):
        rc = P.lib.pdssm_scan_fwd_multi(ctypes.byref(d), chunk, n_out, *args(0))
        assert rc == want, (n_out, chunk, rc, P.lib.pdssm_last_error())
    # the general scan takes several outputs too (N = 17): here it stops at the empty workspace,
    # and past its on-chip budget (N = 64, four outputs at chunk 512) the shape is unsupported
    d17 = _dims(P, L=4096, N=17)
    assert P.lib.pdssm_scan_fwd_multi(ctypes.byref(d17), 128, 2, *args(0)) == -3
    d64 = _dims(P, L=4096, N=64, K=32)
    assert P.lib.pdssm_scan_fwd_multi(ctypes.byref(d64), 512, 4, *args(0)) == -2
    rc = P.lib.pdssm_fwd_wb_multi(ctypes.byref(d), 512, 2, A, A + big, A + 2 * big, A + 3 * big,
                                  A + 4 * big, A + 5 * big, A + 6 * big, None, None, None, A + 7 * big,
                                  A + 8 * big, A + 9 * big, 0, None)
    assert rc == -2
    rc = P.lib.pdssm_fwd_wb_multi(ctypes.byref(d), 128, 4, A, A + big, A + 2 * big, A + 3 * big,
                                  A + 4 * big, A + 5 * big, A + 6 * big, None, None, None, A + 7 * big,
                                  A + 8 * big, A + 9 * big, 0, None)
    assert rc == -3


def test_workspace_status_validation(P):
    """pdssm_workspace_status: NULL or misaligned pointers are invalid, a
    buffer shorter than the 256-byte header is a workspace error; all are
    rejected before anything is enqueued."""
    st = A + (10 << 30)
    fn = P.lib.pdssm_workspace_status
    assert fn(None, 4096, st, None) == -1 and b"workspace" in P.lib.pdssm_last_error()
    assert fn(A, 4096, None, None) == -1 and b"status" in P.lib.pdssm_last_error()
    assert fn(A + 8, 4096, st, None) == -1 and b"aligned" in P.lib.pdssm_last_error()
    assert fn(A, 4096, st + 2, None) == -1 and b"aligned" in P.lib.pdssm_last_error()
    assert fn(A, 255, st, None) == -3 and b"header" in P.lib.pdssm_last_error()


def test_noalloc_validation(P):
    """The allocation-free entry point validates like pdssm_fwd and refuses,
    before any HIP call, a call whose look-back scratch would exceed its
    per-device array."""
    big = 1 << 30
    fn = P.lib.pdssm_fwd_noalloc
    d = _dims(P, B=8, L=131072)                      # 256 chunks x 256 sequences: 32 MiB of scratch
    assert P.fwd_workspace_bytes(d, 512) > P.PDSSM_NOALLOC_SCRATCH_BYTES
    args = [A, A + big, A + 2 * big, A + 3 * big, A + 4 * big, A + 5 * big, A + 6 * big, None, None, None,
            A + 7 * big, A + 8 * big, None, None]
    assert fn(ctypes.byref(d), 512, *args) == -2 and b"scratch" in P.lib.pdssm_last_error()
    d = _dims(P, L=2048)
    bad = list(args)
    bad[5] = None                                    # Bu
    assert fn(ctypes.byref(d), 128, *bad) == -1 and b"Bu" in P.lib.pdssm_last_error()
    bad = list(args)
    bad[12] = A + 9 * big + 2                        # misaligned status
    assert fn(ctypes.byref(d), 128, *bad) == -1 and b"status" in P.lib.pdssm_last_error()
    bad = list(args)
    bad[12] = A + 7 * big                            # status inside y
    assert fn(ctypes.byref(d), 128, *bad) == -1 and b"overlaps" in P.lib.pdssm_last_error()


def test_workspace_query_accepts_shapes_only_the_folded_plans_hold(P):
    """The fused workspace size depends only on the chunk count, and the
    query accepts a shape when any fused call can run it: the LM-layer shape
    at chunk 256 exceeds pdssm_fwd's on-chip budget but not that of the
    folded general kernel (one workgroup per compute unit)."""
    d = P.make_dims(16, 24, 2048, 64, 32, 768, True, True)
    n = P.fwd_workspace_bytes(d, 256)
    assert n == 256 + 8 * 16 * 24 * 4 * 64 * 8
    assert P.lib.pdssm_last_error() == b""


def test_two_pass_workspace_and_validation(P):
    """u shared by the heads in bf16 with N = 64 (the multi-head layer shape)
    runs pdssm_fwd as two passes: the workspace query adds room for k*, D
    and the drive term beyond the scan's look-back words, a workspace of
    only the fused kernel's size is rejected, and the argument checks run
    before any launch."""
    B, H, L, N, K, d = 2, 3, 1000, 64, 32, 768
    dims = P.make_dims(B, H, L, N, K, d, True, True)
    n = P.fwd_workspace_bytes(dims, 96)
    look = P.scan_workspace_bytes(dims, 96)
    assert n >= look + B * H * L * (2 * N + 1) * 4
    big = 1 << 30
    args = dict(dims=dims, chunk=96, u=A, W_sel=A + big, dict_idx=A + 2 * big, W_d=A + 3 * big,
                b_d=A + 4 * big, Bu=A + 5 * big, C=A + 6 * big, h0=None, k_star=None, D=None,
                y=A + 7 * big, h_L=A + 8 * big, ws=A + 9 * big, ws_bytes=look, stream=None)
    assert _call_fwd(P, args) == -3                      # the fused kernel's size is not enough here
    assert b"workspace" in P.lib.pdssm_last_error()
    args["ws_bytes"] = n
    args["Bu"] = None
    assert _call_fwd(P, args) == -1                      # Bu is required on this route too
    args["Bu"] = A + 5 * big
    args["y"] = A + 5 * big + 64                         # y inside Bu
    assert _call_fwd(P, args) == -1
    assert b"overlaps" in P.lib.pdssm_last_error()

"""ctypes loader for libpdscan.so and the C ABI's types and status codes
(see include/pdscan.h)."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpdscan.so")

PDSSM_OK = 0
PDSSM_EINVAL = -1
PDSSM_EUNSUPPORTED = -2
PDSSM_EWORKSPACE = -3
PDSSM_EHIP = -4
PDSSM_F32 = 0
PDSSM_BF16 = 1
PDSSM_NOALLOC_SCRATCH_BYTES = 16 << 20


class PdssmDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "L", "N", "K", "d_in", "u_shared", "in_dtype")]


class PdssmError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"libpdscan status {status}: {message}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -m structured_sparse_state_pdssm_amd.build)")
    # PyTorch ships its own HIP runtime (same soname as the system one).  It
    # must be loaded first so that this library binds to that one runtime:
    # device pointers and streams come from torch.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(PdssmDims)
    sig = {
        "pdssm_select": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "pdssm_scan_workspace_bytes": [dp, i32, ctypes.POINTER(sz)],
        "pdssm_scan_fwd": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_fwd_workspace_bytes": [dp, i32, ctypes.POINTER(sz)],
        "pdssm_fwd": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_fwd_wb": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_fwd_wb_multi": [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_scan_fwd_multi": [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_impulse_sens_workspace_bytes": [dp, i32, ctypes.POINTER(sz)],
        "pdssm_impulse_sens": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_scan_fwd_pidx": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_soft_select": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "pdssm_dict_hardmax": [i32, i32, i32, vp, vp, vp],
        "pdssm_scan_states": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_scan_bwd_workspace_bytes": [dp, i32, ctypes.POINTER(sz)],
        "pdssm_scan_bwd": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "pdssm_status_str": [ctypes.c_int],
        "pdssm_last_error": [],
        "pdssm_abi_version": [],
        "pdssm_workspace_status": [vp, sz, vp, vp],
        "pdssm_fwd_noalloc": [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pdssm_status_str.restype = ctypes.c_char_p
    lib.pdssm_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()

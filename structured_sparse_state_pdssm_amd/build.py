"""Build libpdscan.so in-tree with hipcc for gfx950.

    python -m structured_sparse_state_pdssm_amd.build [--verbose] [--save-temps DIR]
"""

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpdscan.so")

SOURCES = ["pdscan_api.cpp", "pdscan_kernels.hip"]
HEADERS = ["pdscan_plan.h"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # packed fp32 VALU forms stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpdscan)")


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every source into libpdscan.so (always recompiles)."""
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, f"-save-temps={'obj'}")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=save_temps or CSRC, capture_output=True, text=True)
    msgs = "\n".join(
        ln for ln in (r.stdout + r.stderr).splitlines()
        if "packed-fp32-ops" not in ln)          # the host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None)
    ns = ap.parse_args()
    print(build(verbose=ns.verbose, save_temps=ns.save_temps))
    sys.exit(0)

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

SOURCES = ["pdscan_api.cpp", "pdscan_launch_select.hip", "pdscan_launch_scan.hip",
           "pdscan_launch_fused.hip", "pdscan_launch_fused16.hip", "pdscan_launch_fused_multi.hip", "pdscan_launch_fused_fold.hip", "pdscan_launch_bwd.hip", "pdscan_launch_sens.hip", "pdscan_launch_soft.hip",
           "pdscan_noalloc.hip", "pdscan_launch_gemm_sel.hip"]
HEADERS = ["pdscan_plan.h", "pdscan_device.h", "pdscan_launch_general.h", "pdscan_bwd_plan.h", "pdscan_bwd.h",
           "pdscan_sens_plan.h", "pdscan_sens.h", "pdscan_soft_plan.h", "pdscan_soft.h", "pdscan_gemm_sel.h", "pdscan_gemm_sel_plan.h"]

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # packed fp32 VALU forms stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
LINK_FLAGS = ["-shared", "-fPIC", "--offload-arch=gfx950"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpdscan)")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)   # the host pass does not know it
    return r.returncode, msgs


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every source (in parallel, one process per translation unit)
    and link libpdscan.so.  Always recompiles."""
    import concurrent.futures as cf
    import tempfile

    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="pdscan_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *COMPILE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if save_temps:
                cmd.insert(1, "-save-temps=obj")
            objs.append(obj)
            cmds.append(cmd)
        cwd = save_temps or tmp
        if save_temps:
            os.makedirs(save_temps, exist_ok=True)
        with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda c: _run(c, cwd), cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}):\n{msgs}")
            if verbose and msgs.strip():
                print(msgs, flush=True)
        out_tmp = LIB + ".tmp"
        rc, msgs = _run([cc, *LINK_FLAGS, *objs, "-o", out_tmp], tmp)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None)
    ns = ap.parse_args()
    print(build(verbose=ns.verbose, save_temps=ns.save_temps))
    sys.exit(0)

"""Host-side validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.  The API source and the plan headers are built
with g++ (host code only, no device code) into a standalone program with
stand-in launchers; it runs every validation case of tests/sanitize (NULL,
misaligned and overlapping pointers, bad dims, short workspaces, unsupported
shapes, workspace-size queries on every benchmark shape and extreme dims)
and fails on any unexpected status, any launcher reached, or any sanitizer
report."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_sparse_state_pdssm_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIP_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INC),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INC}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "pdscan_api.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
           os.path.join(SAN, "abi_validation.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("PDSSM_TEST_LOOKBACK_GIVEUP", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "ok: 0 failures" in r.stdout, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report

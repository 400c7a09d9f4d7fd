"""Host logic of bench.py, no GPU: the one-GPU rule, the algorithmic byte
counts against sums written out by hand for the impulse shape, and the
counter-to-traffic arithmetic on synthetic counter files."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_impulse_shape(bench):
    from pdssm_inputs import get_config
    c = get_config("impulse")
    steps = 1 * 32 * 131072
    params = 32 * 8 * 64 * 4 + 32 * 16 * 64 * 4 + 32 * 16 * 4 + 32 * 8 * 16 * 4 + 32 * 16 * 4
    # u (64 fp32) + Bu (16 fp32) + y per step, h0 and h_L per sequence
    fwd, flops = bench.algorithmic(c)
    assert fwd == steps * (256 + 64 + 4) + 2 * 32 * 16 * 4 + params == 1359175680
    assert flops == 2 * (8 + 16) * 64 * steps
    # folded: no Bu, W_b read, N more GEMM columns
    fold, fflops = bench.algorithmic(c, fold=True)
    assert fold == steps * (256 + 4) + 2 * 32 * 16 * 4 + params + 32 * 16 * 64 * 4
    assert fflops == 2 * (8 + 32) * 64 * steps
    # gradient: k*, D, g_y, h_t read; dBu, dD written
    assert bench.algorithmic_bwd(c) == steps * (4 + 64 + 4 + 64 + 64 + 64) + (32 * 8 * 16 + 2 * 32 * 16 + 3 * 32 * 16) * 4
    # sensitivity: k*, D read, dY written
    assert bench.algorithmic_sens(c) == steps * (4 + 64 + 256) + (32 * 8 * 16 + 32 * 16 + 2 * 32 * 16 * 64 + 32 * 16) * 4
    # soft: u read, M_t / P_idx / D written, P_idx / D / Bu read, y written
    soft = bench.algorithmic_soft(c)
    assert soft == (steps * (256 + 1024 + 128 + 128 + 64 + 4)
                    + (32 * 8 * 64 + 32 * 16 * 64 + 32 * 16 + 32 * 8 * 256 + 32 * 16 + 2 * 32 * 16) * 4)


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Dispatch_Id"])
        w.writeheader()
        for i, (k, n, v) in enumerate(rows):
            w.writerow({"Kernel_Name": k, "Counter_Name": n, "Counter_Value": v, "Dispatch_Id": i})


def test_traffic_from_counters(bench, tmp_path, monkeypatch):
    """The copy probe reads 1 GiB and writes 1 GiB; its FETCH_SIZE reads back
    half and WRITE_SIZE all of it, so the kernel's counts are scaled by 2 and
    1.  Two kernels of one call (the soft path) add."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    gib_kib = bench.COPY_PROBE_BYTES / 1024.0
    probe = "void at::native::neg_kernel"
    _write_counters(str(tmp_path / "f"), [(probe, "FETCH_SIZE", gib_kib / 2),
                                         ("void pdscan::pdssm_soft_kernel<16>(x)", "FETCH_SIZE", 1000.0),
                                         ("void pdscan::pdssm_soft_kernel<16>(x)", "FETCH_SIZE", 1200.0),
                                         ("void pdscan::pdssm_step16_kernel<1, 1, 0>(x)", "FETCH_SIZE", 300.0),
                                         ("pdscan::clear_kernel(x)", "FETCH_SIZE", 5.0)])
    _write_counters(str(tmp_path / "w"), [(probe, "WRITE_SIZE", gib_kib),
                                         ("void pdscan::pdssm_soft_kernel<16>(x)", "WRITE_SIZE", 4000.0),
                                         ("void pdscan::pdssm_step16_kernel<1, 1, 0>(x)", "WRITE_SIZE", 10.0)])
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), "unit", "soft")
    rec = json.load(open(tmp_path / "profiles" / "pdssm_soft_unit_traffic.json"))
    c = rec["counters"]
    assert c["FETCH_SIZE"]["scale"] == pytest.approx(2.0) and c["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert c["FETCH_SIZE"]["bytes"] == pytest.approx((1100.0 + 300.0) * 1024 * 2)
    assert c["WRITE_SIZE"]["bytes"] == pytest.approx((4000.0 + 10.0) * 1024)
    assert rec["hbm_bytes_per_launch"] == round((1400.0 * 2 + 4010.0) * 1024)

"""Host logic of the launch plans (no GPU): the plan header compiled with
g++ into a small driver (tests/sanitize/plan_choices.cpp) that prints the
dispatcher's choices for the benchmark shapes.

Checked: which kernel takes each workload (the step-major N <= 16 kernel for
the impulse and base shapes, the step-major N = 32 selection tiles for the
time-series shape at chunk <= 256, the general kernel otherwise, and the
deep selection's weight stages: 64-channel blocks unfolded, 32 folded), the on-chip
budgets (64 KiB, or 160 KiB for the folded and multi-output general plans,
with the folded LM-layer plan at chunk 96 small enough for two workgroups
per CU), and the die grouping's choice of head groups: two for the LM-layer
shape (shared u: fetched twice, the weights of 12 heads per die stay in
L2), four when its drive is folded (the weights of 12 heads would exceed the
per-die budget), none for per-head inputs with small weights, and none when
a class of dies would be empty at one batch and eight head groups are not
possible either."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_sparse_state_pdssm_amd", "csrc")


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_choices")
    r = subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}",
                        os.path.join(ROOT, "tests", "sanitize", "plan_choices.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        name, *kv = line.split()
        out[name] = {k: int(v) for k, v in (x.split("=") for x in kv)}
    return out


def test_kernel_choice(plans):
    assert plans["impulse"]["fused16"] == 1 and plans["base"]["fused16"] == 1
    # the step-major kernel takes at most 32 steps per lane group (chunk 512);
    # longer chunks of the same shapes go to the general kernel
    assert plans["impulse"]["S"] == 32 and 3 * plans["impulse"]["lds"] <= 160 * 1024
    for name in ("impulse_c640", "impulse_c768", "impulse_c640_p2"):
        assert plans[name]["ok"] == 1 and plans[name]["fused16"] == 0, name
    ts = plans["timeseries"]
    assert ts["fused16"] == 0 and ts["step32"] == 1 and ts["gse"] == 1
    assert ts["S"] == 32 and ts["G"] == 8                      # two 16-step tiles per group
    assert plans["timeseries_k17"]["step32"] == 0              # more scores than a 16-lane row
    assert plans["timeseries_fold"]["step32"] == 0 and plans["timeseries_fold"]["fold"] == 1
    assert plans["timeseries_c512"]["ok"] == 0                 # [32][516] fp32 rows exceed 64 KiB
    # the LM-layer selection stages its weights in 64-channel blocks (whole
    # 128-byte lines); folded, its ten column tiles keep 32-channel stages
    assert plans["lm_layer"]["step32"] == 0 and plans["lm_layer"]["wst"] == 2
    assert plans["lm_layer_fold"]["wst"] == 1
    # the GPU edge cases of the deep path take the stage variant they name
    assert plans["edge_d320"]["wst"] == 2 and plans["edge_d384"]["wst"] == 2
    assert plans["edge_d800"]["wst"] == 1                     # d not a multiple of 64


def test_on_chip_budgets(plans):
    assert plans["lm_layer"]["limit"] == 64 * 1024 and plans["lm_layer"]["lds"] <= 64 * 1024
    for k in ("lm_layer_fold", "lm_layer_fold_c128", "lm_layer_multi"):
        assert plans[k]["ok"] == 1 and plans[k]["limit"] == 160 * 1024
    # two workgroups per CU at chunk 96 (and for two outputs at chunk 64), one at 128
    assert 2 * plans["lm_layer_fold"]["lds"] <= 160 * 1024
    assert 2 * plans["lm_layer_multi"]["lds"] <= 160 * 1024
    assert 2 * plans["lm_layer_fold_c128"]["lds"] > 160 * 1024


def test_die_grouping_choice(plans):
    lm = plans["lm_layer"]
    assert lm["hg"] == 2 and lm["tasks"] == lm["plain"]        # 8 classes of 4 batches x 12 heads, no padding
    assert plans["lm_layer_fold"]["hg"] == 4
    assert plans["timeseries"]["hg"] == 0
    small = plans["lm_small"]                                  # B = 3, H = 5: padded classes
    assert small["hg"] == 4 and small["tasks"] >= small["plain"]
    assert plans["lm_b1"]["hg"] == 8                           # one batch: only head groups fill the dies
    # per-head inputs whose weights pass 1 MiB (96 heads of 48 x 128 bf16):
    # the step-major N = 32 path, grouped by heads
    h96 = plans["timeseries_h96"]
    assert h96["step32"] == 1 and h96["hg"] == 8

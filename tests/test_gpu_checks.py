"""GPU checks of the timed kernels beyond the parity suite:

* argmax ties through the fused pass itself (the step-major kernel with the
  fp32 three-piece split and with bf16 products, and the general kernel's
  register-resident and deep selections): the lowest index must win;
* run-to-run bit identity of the general kernel on the time-series and
  LM-layer shapes (many chunks, so the look-back is exercised), and bit
  identity across its groupings of the sequences over the dies;
* score accuracy of the three-piece split on inputs whose channels span a
  wide exponent range, and on products of values near the bottom of the
  normal range, against the fp64 definition;
* the look-back status word: a call whose waits are made to give up (a host
  test hook: every wait ignores the carries it finds and stops after two
  reads, so every kernel still ends normally) reports a nonzero status
  through pdssm_workspace_status, and a normal call afterwards reports zero.
"""


import numpy as np
import pytest

import oracle
from pdssm_inputs import bf16_round, generate, get_config
from tests._gpu import assert_within, host, lib, proj_dev, run_fwd, to_dev, torch_mod, upload

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------
# ties through pdssm_fwd
# ----------------------------------------------------------------------------

TIE_SHAPES = [
    # (label, u_shared, bf16, B, H, L, N, K, d, chunk)
    ("fused16 fp32 split d=64", False, False, 1, 4, 1500, 16, 8, 64, 512),
    ("fused16 fp32 split d=32", False, False, 2, 2, 700, 16, 8, 32, 128),
    ("fused16 bf16 d=128", False, True, 1, 4, 1500, 16, 8, 128, 512),
    ("general bf16 d=128 N=32", False, True, 2, 2, 600, 32, 16, 128, 256),
    ("general bf16 shared d=768 N=64", True, True, 2, 5, 300, 64, 32, 768, 128),
    ("general bf16 shared d=768 N=32", True, True, 2, 3, 300, 32, 16, 768, 128),
]


@pytest.mark.parametrize("shape", TIE_SHAPES, ids=[s[0] for s in TIE_SHAPES])
def test_argmax_ties_through_fused_pass(shape):
    """Rows 2 and 6 of W_sel are identical and give the largest score at
    every step, so every selection must be 2 (ties go to the lowest index;
    identical operands give identical fp32 sums on every path)."""
    label, shared, bf, B, H, L, N, K, d, chunk = shape
    rng = np.random.default_rng(91)
    ush = (B, L, d) if shared else (B, H, L, d)
    u = (rng.standard_normal(ush) * 0.1).astype(np.float32)
    u[..., 0] = np.abs(u[..., 0]) + 1.0
    W = (rng.standard_normal((H, K, d)) * 0.01).astype(np.float32)
    W[:, 2] = 0
    W[:, 2, 0] = 5.0
    W[:, 6] = W[:, 2]
    Wd = (rng.standard_normal((H, N, d)) / np.sqrt(d)).astype(np.float32)
    if bf:
        u, W, Wd = bf16_round(u), bf16_round(W), bf16_round(Wd)
    dic = rng.integers(0, N, (H, K, N)).astype(np.int32)
    Bu = rng.standard_normal((B, H, L, N)).astype(np.float32)
    C = (rng.standard_normal((H, N)) / np.sqrt(N)).astype(np.float32)
    b_d = np.full((H, N), 2.0, np.float32)
    P = lib()
    print(f"[gpu] ties through pdssm_fwd: {label}", flush=True)
    out = P.pdssm_fwd(proj_dev(u, bf), proj_dev(W, bf), to_dev(dic), proj_dev(Wd, bf), to_dev(b_d),
                      to_dev(Bu), to_dev(C), None, chunk=chunk, want_k=True)
    k = host(out["k_star"])
    assert (k == 2).all(), f"{label}: {(k != 2).sum()} selections are not the lower tied index"
    assert np.isfinite(host(out["y"])).all()


# ----------------------------------------------------------------------------
# run-to-run bit identity of the general kernel
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,kw", [
    ("timeseries", dict(B=2, H=4, L=4096)),
    ("lm_layer", dict(B=4, H=24, L=2048)),
])
def test_general_kernel_bit_identical_runs(name, kw):
    inp = generate(get_config(name, **kw))
    dev = upload(inp)
    chunk = inp.cfg.chunk
    print(f"[gpu] determinism {name} {kw}", flush=True)
    runs = [run_fwd(dev, chunk) for _ in range(3)]
    for key in ("y", "h_L", "k_star", "D"):
        a = host(runs[0][key])
        for r in runs[1:]:
            assert np.array_equal(a, host(r[key])), f"{name}: {key} differs between runs"


# ----------------------------------------------------------------------------
# die grouping of the general fused kernel
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,kw", [
    ("lm_layer", dict(B=8, H=8, L=300)),           # u shared; every grouping possible
    ("lm_layer", dict(B=3, H=5, L=260, N=32, K=16)),   # ragged groups, padded classes
    ("timeseries", dict(B=8, H=8, L=600, d=512)),  # u per head, weights of 1.5 MiB
    ("timeseries", dict(B=1, H=96, L=520)),        # step-major N = 32 tiles; grouped by default (hg = 8)
])
def test_die_grouping_does_not_change_results(name, kw, monkeypatch):
    """The general kernel's (b, h) grouping over the dies (forced through the
    PDSSM_XCD_HEAD_GROUPS hook; a grouping that would leave a die class empty
    falls back to none) changes only which workgroup runs which task: every
    output is bit-identical to the ungrouped order, and within the tolerance
    of the oracle."""
    inp = generate(get_config(name, **kw))
    ref = oracle.forward_inputs(inp)
    dev = upload(inp)
    chunk = inp.cfg.chunk
    outs = {}
    for hg in ("0", "1", "2", "4", "8"):
        monkeypatch.setenv("PDSSM_XCD_HEAD_GROUPS", hg)
        print(f"[gpu] die grouping {name} {kw} head groups {hg}", flush=True)
        outs[hg] = run_fwd(dev, chunk)
    monkeypatch.delenv("PDSSM_XCD_HEAD_GROUPS")
    print(f"[gpu] die grouping {name} {kw} default", flush=True)
    outs["default"] = run_fwd(dev, chunk)
    base = {k: host(v) for k, v in outs["0"].items()}
    assert np.array_equal(base["k_star"], ref["k_star"])
    assert_within(base["y"], ref["y"], f"{name} y")
    assert_within(base["h_L"], ref["h_L"], f"{name} h_L")
    for hg, o in outs.items():
        for key in ("y", "h_L", "k_star", "D"):
            assert np.array_equal(base[key], host(o[key])), f"{name}: {key} differs with head groups {hg}"


# ----------------------------------------------------------------------------
# three-piece split accuracy on wide exponent ranges
# ----------------------------------------------------------------------------

def _scaled_inputs(rng, B, H, L, N, K, d, eu, ew):
    """u[..., c] = m 2^eu[c], W[..., c] = w 2^ew[c]: every product is
    (m w) 2^(eu + ew); fp32 values, exact powers of two as scales."""
    m = rng.standard_normal((B, H, L, d))
    u = np.ldexp(m, eu).astype(np.float32)
    W = np.ldexp(rng.standard_normal((H, K, d)) / np.sqrt(d), ew).astype(np.float32)
    Wd = np.ldexp(rng.standard_normal((H, N, d)) / np.sqrt(d), ew).astype(np.float32)
    return u, W, Wd


@pytest.mark.parametrize("case", ["mixed_2pow20", "near_min_normal"])
def test_split_accuracy_wide_range(case):
    """Scores and pre-activations of the fp32 step-major kernel (products on
    the bf16 matrix cores from exact three-piece splits) against the fp64
    definition.  Bound: each product keeps the pieces of weight >= 2^-16,
    so |error| <= 2^-22 sum_c |u_c w_c| per score (dropped pieces plus fp32
    accumulation); selections must match wherever the fp64 top-2 gap exceeds
    twice that bound, and |D - D_ref| <= 2e-6 everywhere.
    mixed_2pow20: channels scaled by 2^+20 or 2^-20 (weights by the inverse).
    near_min_normal: u ~ 2^-110, W ~ 2^+100, so the smallest piece of u sits
    at the bottom of the normal range (2^-126) and below it."""
    rng = np.random.default_rng(5 if case == "mixed_2pow20" else 6)
    B, H, L, N, K, d, chunk = 1, 4, 1024, 16, 8, 64, 512
    if case == "mixed_2pow20":
        e = np.where(rng.random(d) < 0.5, 20, -20)
        eu, ew = e, -e
    else:
        eu = np.full(d, -110) + rng.integers(-6, 3, d)
        ew = np.full(d, 100)
    u, W, Wd = _scaled_inputs(rng, B, H, L, N, K, d, eu, ew)
    b_d = np.full((H, N), 0.5, np.float32)
    dic = rng.integers(0, N, (H, K, N)).astype(np.int32)
    Bu = rng.standard_normal((B, H, L, N)).astype(np.float32)
    C = (rng.standard_normal((H, N)) / 4).astype(np.float32)
    s = np.einsum("bhlc,hkc->bhlk", u.astype(np.float64), W.astype(np.float64))
    z = np.einsum("bhlc,hnc->bhln", u.astype(np.float64), Wd.astype(np.float64)) + b_d[None, :, None, :]
    mag = np.einsum("bhlc,hkc->bhlk", np.abs(u.astype(np.float64)), np.abs(W.astype(np.float64)))
    bound = 2.0 ** -22 * mag.max(-1)
    top2 = np.sort(s, -1)[..., -2:]
    clear = (top2[..., 1] - top2[..., 0]) > 2 * bound
    assert clear.mean() > 0.9
    P = lib()
    print(f"[gpu] split accuracy {case}", flush=True)
    out = P.pdssm_fwd(to_dev(u), to_dev(W), to_dev(dic), to_dev(Wd), to_dev(b_d), to_dev(Bu), to_dev(C), None,
                      chunk=chunk, want_k=True, want_D=True)
    k = host(out["k_star"])
    want = np.argmax(s, -1)
    assert (k[clear] == want[clear]).all(), f"{case}: {(k[clear] != want[clear]).sum()} selections differ"
    D_ref = 1.0 / (1.0 + np.exp(-z))
    err = np.abs(host(out["D"]) - D_ref).max()
    assert err <= 2e-6, f"{case}: D error {err:.3g}"


# ----------------------------------------------------------------------------
# look-back status through the C ABI
# ----------------------------------------------------------------------------

@pytest.fixture
def giveup(monkeypatch):
    """The library reads the hook at every call; monkeypatch restores the
    environment after the test."""
    monkeypatch.setenv("PDSSM_TEST_LOOKBACK_GIVEUP", "1")


def _fwd_with_ws(P, dev, inp, chunk):
    c = inp.cfg
    dims = P.make_dims(c.B, c.H, c.L, c.N, c.K, c.d, c.u_shared, c.dtype == "bf16")
    ws = torch_mod().empty(P.fwd_workspace_bytes(dims, chunk), dtype=torch_mod().uint8, device="cuda")
    out = run_fwd(dev, chunk, workspace=ws)
    return out, ws


@pytest.mark.parametrize("name,kw", [("base", dict(B=2, H=3, L=700)), ("timeseries", dict(B=1, H=2, L=1200))])
def test_lookback_status_reports_a_forced_giveup(name, kw, giveup, monkeypatch):
    inp = generate(get_config(name, **kw))
    ref = oracle.forward_inputs(inp)
    dev = upload(inp)
    P = lib()
    chunk = 128
    print(f"[gpu] forced look-back give-up {name}", flush=True)
    out, ws = _fwd_with_ws(P, dev, inp, chunk)
    acc = P.pdssm_workspace_status(ws)
    assert int(host(acc)[0]) != 0, "a forced give-up must set the status word"
    # the chunks after the first continued from h0, so y differs from the oracle there
    assert not np.allclose(host(out["y"])[..., chunk:], ref["y"][..., chunk:], rtol=1e-4, atol=1e-4)
    # a normal call on the same workspace clears the word; the accumulator keeps the earlier one
    monkeypatch.delenv("PDSSM_TEST_LOOKBACK_GIVEUP")
    out2 = run_fwd(dev, chunk, workspace=ws)
    fresh = P.pdssm_workspace_status(ws)
    assert int(host(fresh)[0]) == 0
    P.pdssm_workspace_status(ws, acc)
    assert int(host(acc)[0]) != 0
    assert_within(host(out2["y"]), ref["y"], f"{name} y after the status check")


def test_lookback_status_gradient_and_sensitivity(giveup):
    """The same word in the gradient pass and the impulse sensitivity."""
    inp = generate(get_config("impulse", H=2, L=1500))
    ref = oracle.forward_inputs(inp)
    P = lib()
    c = inp.cfg
    dims = P.make_dims(c.B, c.H, c.L, c.N, c.K, c.d)
    k, dic = to_dev(ref["k_star"]), to_dev(inp.dict_idx)
    D = to_dev(ref["D"].astype(np.float32))
    H_all = to_dev(np.zeros((c.B, c.H, c.L, c.N), np.float32))
    g_y = to_dev(np.ones((c.B, c.H, c.L), np.float32))
    ws = torch_mod().empty(P.scan_bwd_workspace_bytes(dims, 512), dtype=torch_mod().uint8, device="cuda")
    print("[gpu] forced give-up: gradient", flush=True)
    P.pdssm_scan_bwd(k, dic, D, to_dev(inp.C), H_all, g_y, chunk=512, workspace=ws)
    assert int(host(P.pdssm_workspace_status(ws))[0]) != 0
    ws2 = torch_mod().empty(P.impulse_sens_workspace_bytes(dims, 512), dtype=torch_mod().uint8, device="cuda")
    print("[gpu] forced give-up: sensitivity", flush=True)
    P.pdssm_impulse_sens(k, dic, D, to_dev(inp.W_d), to_dev(inp.W_b), to_dev(inp.C), chunk=512, workspace=ws2)
    assert int(host(P.pdssm_workspace_status(ws2))[0]) != 0

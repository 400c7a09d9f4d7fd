"""Parity of the several-outputs-per-head paths (``pdssm_scan_fwd_multi``,
``pdssm_fwd_wb_multi``; HIP through the C ABI) with the fp64 oracle
(``scan_multi``, ``forward_wb_multi``).

Bar: k* bit-exact; y and h_L within 1e-4 (1 + |ref|) elementwise."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config, launch_chunk
from tests._gpu import assert_within, host, lib, proj_dev, to_dev

pytestmark = pytest.mark.gpu

# (workload, overrides, n_out, chunk): every chunk here is the longest the
# per-output on-chip rows allow for that n_out, or shorter; ragged last chunks
CASES = {
    "impulse_p2": ("impulse", dict(H=3, L=1300), 2, 256),
    "impulse_p4": ("impulse", dict(H=3, L=1300), 4, 128),
    "impulse_p3_c100": ("impulse", dict(H=2, L=777), 3, 100),
    # past the step-major kernel's 512 steps: the general kernel
    "impulse_p2_c640": ("impulse", dict(H=2, L=1300), 2, 640),
    "base_d32_p2": ("base", dict(B=2, H=2, L=700, d=32), 2, 128),
    "tiny_p4": ("tiny", dict(L=250), 4, 64),
    "bf16_d128_p2": ("timeseries", dict(B=1, H=2, L=600, N=16, K=8), 2, 256),
    "n5_p3": ("base", dict(B=1, H=2, L=333, N=5, K=3), 3, 128),
    # the general kernel: time-series (N = 32) and LM-layer (N = 64, shared
    # u) shapes, an odd N with fp32 inputs
    "timeseries_p2": ("timeseries", dict(B=2, H=2, L=600), 2, 256),
    "timeseries_p3_c128": ("timeseries", dict(B=1, H=2, L=500), 3, 128),
    "lm_layer_p2": ("lm_layer", dict(B=2, H=3, L=300), 2, 128),
    "lm_layer_p4_c64": ("lm_layer", dict(B=1, H=3, L=300), 4, 64),
    "n20_p2": ("base", dict(B=1, H=2, L=333, N=20, K=5, d=24), 2, 100),
}

_cache = {}


def _case(key):
    if key not in _cache:
        name, kw, P, chunk = CASES[key]
        inp = generate(get_config(name, **kw))
        rng = np.random.default_rng(100 + P)
        C = (rng.standard_normal((inp.cfg.H, P, inp.cfg.N)) / np.sqrt(inp.cfg.N)).astype(np.float32)
        ref = oracle.forward_wb_multi(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, C,
                                      inp.h0, inp.cfg.u_shared)
        _cache[key] = (inp, C, chunk, ref)
    return _cache[key]


@pytest.mark.parametrize("key", list(CASES))
def test_fwd_wb_multi_parity(key):
    inp, C, chunk, ref = _case(key)
    bf = inp.cfg.dtype == "bf16"
    P = lib()
    print(f"[gpu] pdssm_fwd_wb_multi {key} n_out={C.shape[1]} chunk={chunk}", flush=True)
    out = P.pdssm_fwd_wb_multi(proj_dev(inp.u, bf), proj_dev(inp.W_sel, bf), to_dev(inp.dict_idx),
                               proj_dev(inp.W_d, bf), to_dev(inp.b_d), proj_dev(inp.W_b, bf), to_dev(C),
                               to_dev(inp.h0), chunk=chunk, want_k=True)
    assert np.array_equal(host(out["k_star"]), ref["k_star"]), f"{key}: k* differs"
    assert_within(host(out["y"]), ref["y"], f"{key} y")
    assert_within(host(out["h_L"]), ref["h_L"], f"{key} h_L")


@pytest.mark.parametrize("key", list(CASES))
def test_scan_multi_parity(key):
    """The scan alone, fed the oracle's selections (D rounded to fp32, which
    the oracle then consumes too) and the fp64 drive rounded to fp32."""
    inp, C, chunk, ref = _case(key)
    D32 = ref["D"].astype(np.float32)
    Bu32 = ref["Bu"].astype(np.float32)
    yr, hr = oracle.scan_multi(ref["k_star"], inp.dict_idx, D32, Bu32, C, inp.h0)
    P = lib()
    print(f"[gpu] pdssm_scan_fwd_multi {key} n_out={C.shape[1]} chunk={chunk}", flush=True)
    y, hL = P.pdssm_scan_fwd_multi(to_dev(ref["k_star"]), to_dev(inp.dict_idx), to_dev(D32), to_dev(Bu32),
                                   to_dev(C), to_dev(inp.h0), chunk=chunk)
    assert_within(host(y), yr, f"{key} y")
    assert_within(host(hL), hr, f"{key} h_L")


def test_single_output_through_the_multi_entry_equals_fwd_wb():
    inp, _, _, _ = _case("impulse_p2")
    P = lib()
    rng = np.random.default_rng(9)
    C1 = rng.standard_normal((inp.cfg.H, 1, inp.cfg.N)).astype(np.float32)
    args = (to_dev(inp.u), to_dev(inp.W_sel), to_dev(inp.dict_idx), to_dev(inp.W_d), to_dev(inp.b_d),
            to_dev(inp.W_b))
    a = P.pdssm_fwd_wb_multi(*args, to_dev(C1), to_dev(inp.h0), chunk=512)
    b = P.pdssm_fwd_wb(*args, to_dev(C1[:, 0]), to_dev(inp.h0), chunk=512)
    assert np.array_equal(host(a["y"])[..., 0], host(b["y"]))
    assert np.array_equal(host(a["h_L"]), host(b["h_L"]))


def test_multi_deterministic():
    inp, C, chunk, _ = _case("impulse_p4")
    P = lib()
    args = (to_dev(inp.u), to_dev(inp.W_sel), to_dev(inp.dict_idx), to_dev(inp.W_d), to_dev(inp.b_d),
            to_dev(inp.W_b), to_dev(C), to_dev(inp.h0))
    a = P.pdssm_fwd_wb_multi(*args, chunk=chunk)
    b = P.pdssm_fwd_wb_multi(*args, chunk=chunk)
    assert np.array_equal(host(a["y"]), host(b["y"])) and np.array_equal(host(a["h_L"]), host(b["h_L"]))


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,P", [("timeseries", 2), ("lm_layer", 2)])
def test_multi_full_size(name, P):
    """Full workloads, two outputs per head, at the benchmark's chunk for the
    multi-output pass (64 on the LM-layer shape, else the workload's)."""
    inp = generate(get_config(name))
    rng = np.random.default_rng(100 + P)
    C = (rng.standard_normal((inp.cfg.H, P, inp.cfg.N)) / np.sqrt(inp.cfg.N)).astype(np.float32)
    ref = oracle.forward_wb_multi(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, C, inp.h0,
                                  inp.cfg.u_shared)
    bf = inp.cfg.dtype == "bf16"
    Pl = lib()
    chunk = min(launch_chunk("multi", inp.cfg), 256)
    print(f"[gpu] pdssm_fwd_wb_multi {name} full size n_out={P} chunk={chunk}", flush=True)
    out = Pl.pdssm_fwd_wb_multi(proj_dev(inp.u, bf), proj_dev(inp.W_sel, bf), to_dev(inp.dict_idx),
                                proj_dev(inp.W_d, bf), to_dev(inp.b_d), proj_dev(inp.W_b, bf), to_dev(C),
                                to_dev(inp.h0), chunk=chunk, want_k=True)
    assert np.array_equal(host(out["k_star"]), ref["k_star"])
    assert_within(host(out["y"]), ref["y"], f"{name} y")
    assert_within(host(out["h_L"]), ref["h_L"], f"{name} h_L")


def test_multi_general_four_outputs_at_chunk_128():
    """LM-layer shape, drive folded, four outputs at chunk 128: the single
    fused kernel would need 182 KB of on-chip rows, more than the 160 KiB of a
    compute unit, and rejects the call when it is the only route; the two-pass
    route (selection and drive GEMMs, then the scan with four rows of C) runs
    it, within the bar of the oracle."""
    import os
    inp = generate(get_config("lm_layer", B=1, H=2, L=256))
    P = lib()
    rng = np.random.default_rng(4)
    C = (rng.standard_normal((inp.cfg.H, 4, inp.cfg.N)) / np.sqrt(inp.cfg.N)).astype(np.float32)
    args = (proj_dev(inp.u, True), proj_dev(inp.W_sel, True), to_dev(inp.dict_idx), proj_dev(inp.W_d, True),
            to_dev(inp.b_d), proj_dev(inp.W_b, True), to_dev(C), to_dev(inp.h0))
    os.environ["PDSSM_FWD_TWO_PASS"] = "0"
    try:
        with pytest.raises(P.PdssmError) as e:
            P.pdssm_fwd_wb_multi(*args, chunk=128)
        assert e.value.status == P.PDSSM_EUNSUPPORTED
    finally:
        del os.environ["PDSSM_FWD_TWO_PASS"]
    print("[gpu] multi lm_layer four outputs chunk 128 (two passes)", flush=True)
    out = P.pdssm_fwd_wb_multi(*args, chunk=128, want_k=True)
    ref = oracle.forward_wb_multi(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, C, inp.h0,
                                  u_shared=True)
    assert np.array_equal(host(out["k_star"]), ref["k_star"])
    assert_within(host(out["y"]), ref["y"], "lm_layer four outputs y")
    assert_within(host(out["h_L"]), ref["h_L"], "lm_layer four outputs h_L")


def test_multi_rejects_a_chunk_too_long_for_its_outputs():
    inp, C, _, _ = _case("impulse_p4")
    P = lib()
    with pytest.raises(P.PdssmError) as e:
        P.pdssm_fwd_wb_multi(to_dev(inp.u), to_dev(inp.W_sel), to_dev(inp.dict_idx), to_dev(inp.W_d),
                             to_dev(inp.b_d), to_dev(inp.W_b), to_dev(C), to_dev(inp.h0), chunk=512)
    assert e.value.status == P.PDSSM_EUNSUPPORTED

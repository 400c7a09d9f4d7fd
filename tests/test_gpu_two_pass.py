"""The forward passes on the multi-head layer shapes that run as two passes
(u shared by the heads in bf16, N > 32: the all-heads selection GEMM, then
the chunked scan), against the fp64 oracle, around the route's edges.

Bars: k* bit-exact, D within 2e-6 (when asked for), y and h_L within
1e-4 (1 + |ref|).  Shapes: N = 48 and 64 (the route), N = 36 (not a multiple
of 4: the single fused kernel), K = 1, 17 and 32, d = 64 and 320, ragged
chunks; the plain, drive-folded and two-output calls; and the two routes
agreeing with each other on the same inputs."""

import os

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config
from tests._gpu import assert_within, host, lib, proj_dev, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, H, L, N, K, d, chunk
    (2, 3, 300, 64, 32, 320, 96),
    (1, 4, 257, 48, 17, 64, 64),
    (2, 2, 200, 64, 1, 64, 128),
    (1, 3, 130, 36, 8, 320, 96),     # N not a multiple of 4: the fused kernel
]
_cache = {}


def _case(B, H, L, N, K, d):
    key = (B, H, L, N, K, d)
    if key not in _cache:
        inp = generate(get_config("lm_layer", B=B, H=H, L=L, N=N, K=K, d=d))
        _cache[key] = inp
    return _cache[key]


def _dev(inp):
    return (proj_dev(inp.u, True), proj_dev(inp.W_sel, True), to_dev(inp.dict_idx), proj_dev(inp.W_d, True),
            to_dev(inp.b_d))


@pytest.mark.parametrize("B,H,L,N,K,d,chunk", SHAPES)
def test_two_pass_forward(B, H, L, N, K, d, chunk):
    inp = _case(B, H, L, N, K, d)
    P = lib()
    u, Ws, dic, Wd, bd = _dev(inp)
    print(f"[gpu] two-pass fwd B={B} H={H} L={L} N={N} K={K} d={d} chunk={chunk}", flush=True)
    out = P.pdssm_fwd(u, Ws, dic, Wd, bd, to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0), chunk=chunk,
                      want_k=True, want_D=True)
    ref = oracle.forward_inputs(inp)
    assert np.array_equal(host(out["k_star"]), ref["k_star"])
    assert np.abs(host(out["D"]) - ref["D"]).max() <= 2e-6
    assert_within(host(out["y"]), ref["y"], "y")
    assert_within(host(out["h_L"]), ref["h_L"], "h_L")
    # without the optional outputs (k* and D in the workspace)
    out2 = P.pdssm_fwd(u, Ws, dic, Wd, bd, to_dev(inp.Bu), to_dev(inp.C), None, chunk=chunk)
    ref0 = oracle.forward(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.Bu, inp.C, None, u_shared=True)
    assert_within(host(out2["y"]), ref0["y"], "y (h0 = 0)")


@pytest.mark.parametrize("B,H,L,N,K,d,chunk", SHAPES[:3])
def test_two_pass_folded_and_two_outputs(B, H, L, N, K, d, chunk):
    inp = _case(B, H, L, N, K, d)
    P = lib()
    u, Ws, dic, Wd, bd = _dev(inp)
    Wb = proj_dev(inp.W_b, True)
    print(f"[gpu] two-pass fold / multi N={N} K={K} d={d}", flush=True)
    out = P.pdssm_fwd_wb(u, Ws, dic, Wd, bd, Wb, to_dev(inp.C), to_dev(inp.h0), chunk=chunk, want_k=True)
    ref = oracle.forward_wb(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, inp.C, inp.h0,
                            u_shared=True)
    assert np.array_equal(host(out["k_star"]), ref["k_star"])
    assert_within(host(out["y"]), ref["y"], "folded y")
    assert_within(host(out["h_L"]), ref["h_L"], "folded h_L")
    rng = np.random.default_rng(N + K)
    C2 = (rng.standard_normal((H, 2, N)) / np.sqrt(N)).astype(np.float32)
    out = P.pdssm_fwd_wb_multi(u, Ws, dic, Wd, bd, Wb, to_dev(C2), to_dev(inp.h0), chunk=chunk)
    ref = oracle.forward_wb_multi(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, C2, inp.h0,
                                  u_shared=True)
    assert_within(host(out["y"]), ref["y"], "two outputs y")
    assert_within(host(out["h_L"]), ref["h_L"], "two outputs h_L")


def test_two_routes_agree():
    """The two-pass route and the single fused kernel on the same inputs:
    k* identical, y within the bar of each other."""
    inp = _case(*SHAPES[0][:6])
    P = lib()
    args = (*_dev(inp), to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0))
    a = P.pdssm_fwd(*args, chunk=96, want_k=True)
    os.environ["PDSSM_FWD_TWO_PASS"] = "0"
    try:
        b = P.pdssm_fwd(*args, chunk=96, want_k=True)
    finally:
        del os.environ["PDSSM_FWD_TWO_PASS"]
    assert np.array_equal(host(a["k_star"]), host(b["k_star"]))
    assert_within(host(a["y"]), host(b["y"]).astype(np.float64), "routes y")

"""Parity of the forward pass with the drive term folded into the selection
GEMM (``pdssm_fwd_wb``, HIP through the C ABI) with the fp64 oracle
(``forward_wb``: Bu = W_b u in fp64, then the sequential scan).

Bar: k* bit-exact; y and h_L within 1e-4 (1 + |ref|) elementwise; D within
2e-6 absolute."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config, launch_chunk
from tests._gpu import assert_within, host, lib, proj_dev, to_dev, torch_mod

pytestmark = pytest.mark.gpu

# shapes of the step-major kernel: fp32 d = 64 (split products), fp32 d = 32,
# fp32 d = 16 (fp32 MFMA), bf16 d = 128 (bf16 MFMA); and of the general
# kernel, where the drive terms are a third column segment of the selection
# GEMM written to an on-chip buffer: the time-series shape (N = 32, bf16
# d = 128, register-resident weights), the LM-layer shape (N = 64, u shared
# by the heads, bf16 d = 768: deep selection with LDS-staged weights, and at
# chunk 64 without the staging), shared fp32 inputs and an odd N (generic
# selection); ragged last chunks
CASES = {
    "impulse": ("impulse", dict(H=3, L=1300)),
    "base": ("base", dict(B=2, H=3, L=700)),
    "base_d32": ("base", dict(B=1, H=2, L=450, d=32)),
    "tiny": ("tiny", dict(L=250)),
    "bf16_d128": ("timeseries", dict(B=1, H=2, L=600, N=16, K=8)),
    "timeseries": ("timeseries", dict(B=2, H=2, L=600)),
    "lm_layer": ("lm_layer", dict(B=2, H=5, L=300)),
    "shared_f32": ("lm_layer", dict(B=2, H=3, L=200, N=16, K=8, d=64, dtype="f32")),
    "odd_n20": ("base", dict(B=1, H=2, L=333, N=20, K=5, d=24)),
    "lm_n32_k16": ("lm_layer", dict(B=1, H=3, L=260, N=32, K=16)),
}

_cache = {}


def _case(key):
    if key not in _cache:
        name, kw = CASES[key]
        inp = generate(get_config(name, **kw))
        ref = oracle.forward_wb(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, inp.C,
                                inp.h0, inp.cfg.u_shared)
        _cache[key] = (inp, ref)
    return _cache[key]


def _dev(inp):
    bf = inp.cfg.dtype == "bf16"
    return dict(u=proj_dev(inp.u, bf), W_sel=proj_dev(inp.W_sel, bf), W_d=proj_dev(inp.W_d, bf),
                W_b=proj_dev(inp.W_b, bf), b_d=to_dev(inp.b_d), dict_idx=to_dev(inp.dict_idx),
                C=to_dev(inp.C), h0=to_dev(inp.h0))


def _run(d, chunk, h0=True, want=True):
    P = lib()
    return P.pdssm_fwd_wb(d["u"], d["W_sel"], d["dict_idx"], d["W_d"], d["b_d"], d["W_b"], d["C"],
                          d["h0"] if h0 else None, chunk=chunk, want_k=want, want_D=want)


def _check(out, ref, what):
    assert np.array_equal(host(out["k_star"]), ref["k_star"]), f"{what}: k* differs"
    assert np.max(np.abs(host(out["D"]) - ref["D"])) <= 2e-6, f"{what}: D"
    assert_within(host(out["y"]), ref["y"], f"{what} y")
    assert_within(host(out["h_L"]), ref["h_L"], f"{what} h_L")


@pytest.mark.parametrize("key", list(CASES))
def test_fold_parity(key):
    inp, ref = _case(key)
    print(f"[gpu] pdssm_fwd_wb {key} chunk={inp.cfg.chunk}", flush=True)
    _check(_run(_dev(inp), inp.cfg.chunk), ref, key)


@pytest.mark.parametrize("chunk", [1, 4, 16, 100, 128, 512, 640])
def test_fold_chunk_independence(chunk):
    inp, ref = _case("impulse")
    print(f"[gpu] pdssm_fwd_wb impulse chunk={chunk}", flush=True)
    _check(_run(_dev(inp), chunk), ref, f"chunk {chunk}")


@pytest.mark.parametrize("key,chunk", [("lm_layer", 64), ("lm_layer", 96), ("lm_layer", 100), ("lm_layer", 32),
                                       ("timeseries", 128), ("timeseries", 64), ("timeseries", 7)])
def test_fold_general_chunk_independence(key, chunk):
    """The general kernel's folded drive at other chunks: the LM-layer shape
    without the LDS weight staging (chunk 64, 32), a ragged chunk (100), and
    the time-series shape at shorter chunks (one ragged: 7)."""
    inp, ref = _case(key)
    print(f"[gpu] pdssm_fwd_wb {key} chunk={chunk}", flush=True)
    _check(_run(_dev(inp), chunk), ref, f"{key} chunk {chunk}")


def test_fold_without_selection_outputs_or_h0():
    inp, _ = _case("base")
    ref = oracle.forward_wb(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, inp.C, None)
    out = _run(_dev(inp), inp.cfg.chunk, h0=False, want=False)
    assert "k_star" not in out and "D" not in out
    assert_within(host(out["y"]), ref["y"], "y")
    assert_within(host(out["h_L"]), ref["h_L"], "h_L")


def test_fold_matches_the_unfolded_pass_on_the_same_drive():
    """Same u, W_b: pdssm_fwd fed the fp64 drive rounded to fp32 agrees with
    pdssm_fwd_wb within the tolerance (and exactly on k*)."""
    inp, ref = _case("impulse")
    P = lib()
    d = _dev(inp)
    a = _run(d, 512)
    b = P.pdssm_fwd(d["u"], d["W_sel"], d["dict_idx"], d["W_d"], d["b_d"],
                    to_dev(ref["Bu"].astype(np.float32)), d["C"], d["h0"], chunk=512, want_k=True)
    assert np.array_equal(host(a["k_star"]), host(b["k_star"]))
    assert_within(host(a["y"]), host(b["y"]), "y vs unfolded")


def test_fold_deterministic():
    inp, _ = _case("base")
    d = _dev(inp)
    a, b = _run(d, 128), _run(d, 128)
    for n in ("y", "h_L", "k_star", "D"):
        assert np.array_equal(host(a[n]), host(b[n])), n


@pytest.mark.parametrize("name,kw", [("lm_layer", dict(B=1, H=2, L=64, K=64)),
                                     ("base", dict(B=1, H=2, L=64, N=64, K=8, d=64))])
def test_fold_rejects_shapes_whose_gemm_does_not_fit(name, kw):
    """Too many columns for the folded selection GEMM: bf16 d = 768 with
    K = 64, N = 64 (12 tiles of 16, the kernel holds 10) and fp32 with
    K + 2N = 136 > 128."""
    P = lib()
    inp = generate(get_config(name, **kw))
    with pytest.raises(P.PdssmError) as e:
        _run(_dev(inp), inp.cfg.chunk)
    assert e.value.status == P.PDSSM_EUNSUPPORTED


def test_fold_general_deterministic():
    inp, _ = _case("lm_layer")
    d = _dev(inp)
    a, b = _run(d, 128), _run(d, 128)
    for n in ("y", "h_L", "k_star", "D"):
        assert np.array_equal(host(a[n]), host(b[n])), n


def test_fold_die_grouping_does_not_change_results(monkeypatch):
    """The folded general pass under every grouping of the sequences over the
    dies (PDSSM_XCD_HEAD_GROUPS; 1 would leave die classes empty at B = 4
    and falls back to none): bit-identical outputs."""
    inp = generate(get_config("lm_layer", B=4, H=8, L=300))
    d = _dev(inp)
    outs = {}
    for hg in ("0", "1", "2", "4", "8"):
        monkeypatch.setenv("PDSSM_XCD_HEAD_GROUPS", hg)
        print(f"[gpu] pdssm_fwd_wb lm_layer head groups {hg}", flush=True)
        outs[hg] = _run(d, inp.cfg.chunk)
    for hg, o in outs.items():
        for n in ("y", "h_L", "k_star", "D"):
            assert np.array_equal(host(outs["0"][n]), host(o[n])), f"{n} differs with head groups {hg}"


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["impulse", "timeseries", "lm_layer"])
def test_fold_full_size(name):
    """Full workloads in the benchmark's launch configuration (its chunk for
    the folded pass: 96 on the LM-layer shape, else the workload's)."""
    torch = torch_mod()
    inp = generate(get_config(name))
    ref = oracle.forward_wb(inp.u, inp.W_sel, inp.dict_idx, inp.W_d, inp.b_d, inp.W_b, inp.C, inp.h0,
                            inp.cfg.u_shared)
    chunk = launch_chunk("fold", inp.cfg)
    print(f"[gpu] pdssm_fwd_wb {name} full size chunk={chunk}", flush=True)
    out = _run(_dev(inp), chunk)
    torch.cuda.synchronize()
    _check(out, ref, f"{name} full")

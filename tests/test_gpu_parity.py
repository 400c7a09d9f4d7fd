"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: selections bit-exact; y and h_L within 1e-4 (1 + |ref|) elementwise;
D within 2e-6 absolute (diagnostic); automata runs bit-exact.
"""

import dataclasses

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config, launch_chunk
from tests._gpu import TOL, assert_within, host, lib, run_fwd, to_dev, torch_mod, upload

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny": dict(L=250),
    "base": dict(B=2, H=3, L=700),
    "timeseries": dict(B=2, H=2, L=600),
    "impulse": dict(H=4, L=1500),
    "lm_layer": dict(B=2, H=5, L=300),
}

_cache = {}


def _case(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        inp = generate(get_config(name, **kw))
        _cache[key] = (inp, oracle.forward_inputs(inp))
    return _cache[key]


def _check_fwd(inp, ref, chunk, what):
    P = lib()
    dev = upload(inp)
    ws_bytes = P.fwd_workspace_bytes(
        P.make_dims(inp.cfg.B, inp.cfg.H, inp.cfg.L, inp.cfg.N, inp.cfg.K, inp.cfg.d,
                    inp.cfg.u_shared, inp.cfg.dtype == "bf16"), chunk)
    ws = torch_mod().empty(ws_bytes, dtype=torch_mod().uint8, device="cuda")
    print(f"[gpu] pdssm_fwd {what} chunk={chunk}", flush=True)
    out = run_fwd(dev, chunk, workspace=ws)
    k = host(out["k_star"])
    assert P.workspace_error_flag(ws) == 0
    mism = int((k != ref["k_star"]).sum())
    assert mism == 0, f"{what}: {mism} selections differ"
    D = host(out["D"])
    assert np.abs(D - ref["D"]).max() <= 2e-6, f"{what}: D error {np.abs(D - ref['D']).max():.3g}"
    assert_within(host(out["y"]), ref["y"], f"{what} y")
    assert_within(host(out["h_L"]), ref["h_L"], f"{what} h_L")
    return out


@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_parity(name):
    inp, ref = _case(name, **REDUCED[name])
    _check_fwd(inp, ref, inp.cfg.chunk, name)


@pytest.mark.parametrize("chunk", [96, 128])
def test_fused_kernel_lm_layer(chunk):
    """pdssm_fwd on the LM-layer shape runs the selection GEMM and the scan as
    two passes; the single fused kernel it replaces there (still the path of
    the allocation-free entry point) stays checked with the two-pass route
    switched off."""
    import os
    inp, ref = _case("lm_layer", **REDUCED["lm_layer"])
    os.environ["PDSSM_FWD_TWO_PASS"] = "0"
    try:
        _check_fwd(inp, ref, chunk, f"lm_layer fused kernel chunk {chunk}")
    finally:
        del os.environ["PDSSM_FWD_TWO_PASS"]


@pytest.mark.parametrize("name", list(REDUCED))
def test_select_standalone(name):
    inp, ref = _case(name, **REDUCED[name])
    P = lib()
    dev = upload(inp)
    print(f"[gpu] pdssm_select {name}", flush=True)
    k, D, Pi = P.pdssm_select(dev["u"], dev["W_sel"], dev["W_d"], dev["b_d"], dev["dict_idx"],
                              want_P=True)
    k = host(k)
    assert np.array_equal(k, ref["k_star"])
    assert np.abs(host(D) - ref["D"]).max() <= 2e-6
    Pi = host(Pi)
    expect = inp.dict_idx[np.arange(inp.cfg.H)[None, :, None], k]
    assert np.array_equal(Pi, expect)


@pytest.mark.parametrize("name", list(REDUCED))
def test_scan_standalone(name):
    """The scan fed the oracle's selections (D rounded to fp32, which the
    oracle then consumes too)."""
    inp, ref = _case(name, **REDUCED[name])
    P = lib()
    D32 = ref["D"].astype(np.float32)
    y_ref, h_ref = oracle.scan(ref["k_star"], inp.dict_idx, D32, inp.Bu, inp.C, inp.h0)
    print(f"[gpu] pdssm_scan_fwd {name}", flush=True)
    y, hL = P.pdssm_scan_fwd(to_dev(ref["k_star"]), to_dev(inp.dict_idx), to_dev(D32),
                             to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0), chunk=inp.cfg.chunk)
    assert_within(host(y), y_ref, f"{name} y")
    assert_within(host(hL), h_ref, f"{name} h_L")


def _skewed_dictionaries(H, N):
    """Column-one-hot entries with rows of every in-degree: all columns into
    row 0, three sources per row, a permutation, and ten sources in row 0
    with rows 1-9 empty."""
    j = np.arange(N)
    one = np.stack([np.zeros(N, np.int64), j // 3, (j * 7) % N, np.where(j < 10, 0, j)])
    return np.broadcast_to(one, (H, 4, N)).astype(np.int32).copy()


@pytest.mark.parametrize("N", [32, 64, 20])
def test_high_in_degree_rows(N):
    """Rows with up to N sources (the gather over inverse rows with N = 32
    takes its second and third rounds; other N scatter): fused forward and
    scan alone against the oracle."""
    cfg = get_config("timeseries", B=2, H=2, L=500, N=N, K=4)
    inp = dataclasses.replace(generate(cfg), dict_idx=_skewed_dictionaries(2, N))
    ref = oracle.forward_inputs(inp)
    _check_fwd(inp, ref, 128, f"skewed dictionaries N={N}")
    P = lib()
    D32 = ref["D"].astype(np.float32)
    y_ref, h_ref = oracle.scan(ref["k_star"], inp.dict_idx, D32, inp.Bu, inp.C, inp.h0)
    print(f"[gpu] pdssm_scan_fwd skewed dictionaries N={N}", flush=True)
    y, hL = P.pdssm_scan_fwd(to_dev(ref["k_star"]), to_dev(inp.dict_idx), to_dev(D32),
                             to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0), chunk=128)
    assert_within(host(y), y_ref, f"skewed N={N} scan y")
    assert_within(host(hL), h_ref, f"skewed N={N} scan h_L")


@pytest.mark.parametrize("chunk", [1, 3, 16, 100, 512, 700])
@pytest.mark.parametrize("name,kw", [("impulse", dict(H=3, L=1300)), ("base", dict(B=1, H=2, L=333, N=5, K=3))])
def test_scan_chunk_independence(name, kw, chunk):
    """Chunks up to 512 with N <= 16 run the step-major scan (maps streamed
    through registers), longer ones the table-driven scan: both agree with
    the sequential oracle."""
    inp, ref = _case(name, **kw)
    P = lib()
    D32 = ref["D"].astype(np.float32)
    y_ref, h_ref = oracle.scan(ref["k_star"], inp.dict_idx, D32, inp.Bu, inp.C, inp.h0)
    print(f"[gpu] pdssm_scan_fwd {name} N={inp.cfg.N} chunk={chunk}", flush=True)
    y, hL = P.pdssm_scan_fwd(to_dev(ref["k_star"]), to_dev(inp.dict_idx), to_dev(D32),
                             to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0), chunk=chunk)
    assert_within(host(y), y_ref, f"{name} chunk {chunk} y")
    assert_within(host(hL), h_ref, f"{name} chunk {chunk} h_L")


def test_scan_deterministic():
    inp, ref = _case("impulse", **REDUCED["impulse"])
    P = lib()
    args = (to_dev(ref["k_star"]), to_dev(inp.dict_idx), to_dev(ref["D"].astype(np.float32)),
            to_dev(inp.Bu), to_dev(inp.C), to_dev(inp.h0))
    a = P.pdssm_scan_fwd(*args, chunk=512)
    b = P.pdssm_scan_fwd(*args, chunk=512)
    assert np.array_equal(host(a[0]), host(b[0])) and np.array_equal(host(a[1]), host(b[1]))


@pytest.mark.parametrize("chunk", [1, 3, 4, 16, 64, 100, 128, 512, 576, 600, 640, 700, 4096])
def test_chunk_size_independence(chunk):
    inp, ref = _case("base", **REDUCED["base"])
    _check_fwd(inp, ref, chunk, f"base chunk {chunk}")


@pytest.mark.parametrize("chunk", [512, 513, 576, 640])
def test_n16_chunks_at_the_step_major_limit(chunk):
    """N = 16 shapes on either side of the step-major kernel's 512-step limit
    (past it the general kernel takes them), on fp32 d = 64 (the three-piece
    split) and bf16 d = 128, with a ragged last chunk."""
    for name, kw in (("impulse", dict(H=3, L=1500)), ("timeseries", dict(B=1, H=2, L=1500, N=16, K=8))):
        inp, ref = _case(name, **kw)
        _check_fwd(inp, ref, chunk, f"N=16 {name} chunk {chunk}")


@pytest.mark.parametrize("chunk", [7, 16, 48, 100, 200, 256])
@pytest.mark.parametrize("kw", [dict(B=1, H=3, L=700), dict(B=2, H=2, L=430, K=5)],
                         ids=["K16", "K5"])
def test_step_major_n32_tiles(kw, chunk):
    """The time-series shape's step-major selection tiles (N = 32, bf16
    d = 128): one or two 16-step tiles per group, last chunks whose wave
    groups hold different step counts (700 and 430 are not multiples of the
    chunk), K below 16 (score columns past K hold the minimum key), k* and D
    written out, against the oracle."""
    inp, ref = _case("timeseries", **kw)
    _check_fwd(inp, ref, chunk, f"step-major N=32 {kw}")


def test_deterministic_runs():
    inp, _ = _case("impulse", **REDUCED["impulse"])
    dev = upload(inp)
    print("[gpu] determinism impulse", flush=True)
    a = run_fwd(dev, 512)
    b = run_fwd(dev, 512)
    for k in ("y", "h_L", "k_star", "D"):
        assert np.array_equal(host(a[k]), host(b[k])), k


# ----------------------------------------------------------------------------
# closed forms and invariants on the GPU
# ----------------------------------------------------------------------------

def _fsa_dev(delta, symbols, start, C):
    from tests.test_oracle_pins import fsa_inputs
    u, W_sel, dic, W_d, b_d, Bu, h0 = fsa_inputs(delta, symbols, start)
    f = lambda x: to_dev(np.asarray(x, np.float32))  # noqa: E731
    return dict(u=f(u), W_sel=f(W_sel), dict_idx=to_dev(dic.astype(np.int32)), W_d=f(W_d),
                b_d=f(b_d), Bu=f(Bu), C=f(C), h0=f(h0))


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("chunk", [4, 64, 512])
def test_fsa_bit_exact(seed, chunk):
    """Automata (one-hot state, D = 1): outputs must be exactly C[q_t]."""
    rng = np.random.default_rng(300 + seed)
    N, K, L = int(rng.integers(3, 17)), int(rng.integers(2, 6)), 2000
    delta = rng.integers(0, N, size=(K, N))
    sy = rng.integers(0, K, size=L)
    start = int(rng.integers(0, N))
    C = rng.standard_normal((1, N)).astype(np.float32)
    dev = _fsa_dev(delta, sy, start, C)
    print(f"[gpu] fsa seed={seed} chunk={chunk} N={N} K={K}", flush=True)
    out = run_fwd(dev, chunk)
    q, qs = start, []
    for s in sy:
        q = delta[s][q]
        qs.append(q)
    assert np.array_equal(host(out["k_star"])[0, 0], sy)
    assert np.array_equal(host(out["y"])[0, 0], C[0, qs])
    onehot = np.zeros(N, np.float32)
    onehot[qs[-1]] = 1
    assert np.array_equal(host(out["h_L"])[0, 0], onehot)


def test_prefix_sum_on_gpu():
    rng = np.random.default_rng(44)
    B, H, L, N = 2, 3, 3000, 16
    Bu = rng.standard_normal((B, H, L, N)).astype(np.float32)
    h0 = rng.standard_normal((B, H, N)).astype(np.float32)
    C = rng.standard_normal((H, N)).astype(np.float32)
    dic = np.broadcast_to(np.arange(N, dtype=np.int32), (H, 2, N)).copy()
    P = lib()
    y, hL = P.pdssm_scan_fwd(to_dev(np.zeros((B, H, L), np.int32)), to_dev(dic),
                             to_dev(np.ones((B, H, L, N), np.float32)), to_dev(Bu), to_dev(C),
                             to_dev(h0), chunk=256)
    states = h0[:, :, None, :].astype(np.float64) + np.cumsum(Bu.astype(np.float64), axis=2)
    assert_within(host(hL), states[:, :, -1], "h_L")
    assert_within(host(y), (states * C[None, :, None, :]).sum(-1), "y")


def test_cyclic_shift_impulse_on_gpu():
    rng = np.random.default_rng(45)
    N, L = 16, 600
    idx = ((np.arange(N) + 1) % N).astype(np.int32)
    d = rng.uniform(0.9, 1.0, size=N).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    C = rng.standard_normal(N).astype(np.float32)
    Bu = np.zeros((1, 1, L, N), np.float32)
    Bu[0, 0, 0] = b
    P = lib()
    y, _ = P.pdssm_scan_fwd(to_dev(np.zeros((1, 1, L), np.int32)), to_dev(idx[None, None]),
                            to_dev(np.broadcast_to(d, (1, 1, L, N)).copy()), to_dev(Bu),
                            to_dev(C[None]), None, chunk=64)
    y = host(y)[0, 0]
    dd = d.astype(np.float64)
    for t in range(L):
        expect = sum(C[(j + t) % N] * np.prod([dd[(j + m) % N] for m in range(t)]) * b[j]
                     for j in range(N))
        assert abs(y[t] - expect) <= TOL * (1 + abs(expect))


def test_linearity_and_resume_on_gpu():
    inp, ref = _case("base", **REDUCED["base"])
    dev = upload(inp)
    P = lib()
    rng = np.random.default_rng(46)
    Bu2 = rng.standard_normal(inp.Bu.shape).astype(np.float32)
    dev2 = dict(dev, Bu=to_dev(inp.Bu + Bu2))
    y12 = host(run_fwd(dev2, 128)["y"])
    y1 = host(run_fwd(dev, 128)["y"])
    y2 = host(run_fwd(dict(dev, Bu=to_dev(Bu2)), 128, h0=False)["y"])
    assert_within(y12, y1 + y2, "linearity", tol=5e-4)
    # resume: [0, L1) then [L1, L) from the returned state
    L1 = 333
    a = P.pdssm_fwd(dev["u"][:, :, :L1].contiguous(), dev["W_sel"], dev["dict_idx"], dev["W_d"],
                    dev["b_d"], dev["Bu"][:, :, :L1].contiguous(), dev["C"], dev["h0"], chunk=128)
    b = P.pdssm_fwd(dev["u"][:, :, L1:].contiguous(), dev["W_sel"], dev["dict_idx"], dev["W_d"],
                    dev["b_d"], dev["Bu"][:, :, L1:].contiguous(), dev["C"], a["h_L"], chunk=128)
    y = np.concatenate([host(a["y"]), host(b["y"])], axis=2)
    assert_within(y, ref["y"], "resumed y")
    assert_within(host(b["h_L"]), ref["h_L"], "resumed h_L")


@pytest.mark.parametrize("bf16,d", [(False, 64), (True, 128), (True, 32)])
def test_argmax_ties_on_gpu(bf16, d):
    """Two identical maximal score rows: the lower index must win (identical
    inputs give identical fp32 scores on both MFMA paths)."""
    rng = np.random.default_rng(47)
    H, K, N, L = 2, 8, 16, 300
    u = rng.standard_normal((1, H, L, d)).astype(np.float32) * 0.1
    u[..., 0] = np.abs(u[..., 0]) + 1.0
    W = (rng.standard_normal((H, K, d)) * 0.01).astype(np.float32)
    W[:, 2] = 0
    W[:, 2, 0] = 5.0
    W[:, 6] = W[:, 2]
    if bf16:
        from pdssm_inputs import bf16_round
        u, W = bf16_round(u), bf16_round(W)
    Wd = (rng.standard_normal((H, N, d)) * 0.1).astype(np.float32)
    if bf16:
        Wd = bf16_round(Wd)
    P = lib()
    from tests._gpu import proj_dev
    k, _ = P.pdssm_select(proj_dev(u, bf16), proj_dev(W, bf16), proj_dev(Wd, bf16),
                          to_dev(np.zeros((H, N), np.float32)))
    assert (host(k) == 2).all()


@pytest.mark.parametrize("shape", [
    dict(B=1, H=1, L=1, N=8, K=4, d=16, chunk=64),
    dict(B=2, H=3, L=77, N=1, K=1, d=8, chunk=16),
    dict(B=1, H=2, L=301, N=5, K=3, d=24, chunk=32),
    dict(B=3, H=2, L=129, N=12, K=7, d=40, chunk=128),
    dict(B=1, H=1, L=1000, N=64, K=32, d=128, chunk=64),
    dict(B=2, H=2, L=300, N=33, K=2, d=256, chunk=100),
    # the largest shapes the library accepts: K + N = 128, d = 8192 (fp32 and
    # the bf16 deep selection path)
    dict(B=1, H=2, L=150, N=64, K=64, d=64, chunk=64),
    dict(B=1, H=1, L=40, N=16, K=16, d=8192, chunk=16),
    dict(B=1, H=1, L=64, N=64, K=64, d=8192, chunk=32, dtype="bf16"),
    # the bf16 deep selection path with K not a multiple of 16 (score tiles
    # padded, then pre-activation tiles) and an odd number of 32-channel blocks
    dict(B=2, H=2, L=300, N=33, K=17, d=256, chunk=100, dtype="bf16"),
    dict(B=1, H=3, L=200, N=20, K=5, d=288, chunk=64, dtype="bf16"),
    dict(B=1, H=2, L=130, N=64, K=3, d=800, chunk=128, dtype="bf16"),
    # the deep path in 64-channel blocks (d a multiple of 64, unfolded, stages
    # in D's region): an odd number of blocks, and a ragged last chunk
    dict(B=1, H=2, L=300, N=64, K=32, d=320, chunk=128, dtype="bf16"),
    dict(B=2, H=1, L=260, N=64, K=16, d=384, chunk=128, dtype="bf16"),
])
def test_edge_shapes(shape):
    chunk = shape.pop("chunk")
    cfg = get_config("base", **shape)
    inp = generate(cfg)
    ref = oracle.forward_inputs(inp)
    _check_fwd(inp, ref, chunk, f"edge {shape}")


@pytest.mark.parametrize("variant", ["shared_f32", "perhead_bf16_small_d"])
def test_layout_variants(variant):
    if variant == "shared_f32":
        cfg = get_config("lm_layer", B=2, H=3, L=200, N=16, K=8, d=64, dtype="f32")
    else:
        cfg = get_config("timeseries", B=1, H=2, L=300, N=16, K=8, d=64)
    inp = generate(cfg)
    ref = oracle.forward_inputs(inp)
    _check_fwd(inp, ref, 64, variant)


def test_h0_none_equals_zeros():
    inp, _ = _case("base", **REDUCED["base"])
    dev = upload(inp)
    a = run_fwd(dev, 128, h0=False)
    b = run_fwd(dict(dev, h0=to_dev(np.zeros_like(inp.h0))), 128)
    assert np.array_equal(host(a["y"]), host(b["y"]))


# ----------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration
# ----------------------------------------------------------------------------

@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "base", "timeseries", "impulse", "lm_layer"])
def test_full_size(name):
    """Every workload at full size, at its own chunk and, where the benchmark
    launches at another (base: 256), at that one too."""
    inp = generate(get_config(name))
    ref = oracle.forward_inputs(inp)
    for chunk in sorted({inp.cfg.chunk, launch_chunk("fwd", inp.cfg)}):
        print(f"[gpu] full {name} chunk={chunk}", flush=True)
        _check_fwd(inp, ref, chunk, f"full {name} chunk {chunk}")

"""Parity of the states scan and of the gradient pass through the scan (HIP,
through the C ABI) with the fp64 oracle (``scan_states``, ``scan_vjp``).

Selections and diagonals come from the oracle on generated inputs and are fed
to both sides; the gradient pass reads the GPU's own forward states.  Bar:
every output within 1e-4 (1 + |ref|) elementwise."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config, upstream_grads
from tests._gpu import assert_within, host, lib, to_dev, torch_mod

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
        k, D, _ = oracle.select(inp.u, inp.W_sel, inp.W_d, inp.b_d, inp.cfg.u_shared)
        D32 = D.astype(np.float32)
        c = inp.cfg
        rng = np.random.default_rng(c.seed + 17)
        h0 = rng.standard_normal((c.B, c.H, c.N)).astype(np.float32)
        g_y, g_hL = upstream_grads(c.B, c.H, c.L, c.N, c.seed)
        _cache[key] = dict(cfg=c, k=k.astype(np.int32), D=D32, Bu=inp.Bu, C=inp.C, h0=h0,
                           dict_idx=inp.dict_idx, g_y=g_y, g_hL=g_hL)
    return _cache[key]


def _dev(cs):
    return {n: to_dev(cs[n]) for n in ("k", "D", "Bu", "C", "h0", "dict_idx", "g_y", "g_hL")}


def _gpu_states(d, chunk, h0=True):
    P = lib()
    return P.pdssm_scan_states(d["k"], d["dict_idx"], d["D"], d["Bu"], d["C"], d["h0"] if h0 else None,
                               chunk=chunk)


def _gpu_bwd(d, H_all, chunk, h0=True, g_hL=True, want_h0=True):
    P = lib()
    return P.pdssm_scan_bwd(d["k"], d["dict_idx"], d["D"], d["C"], H_all, d["g_y"],
                            h0=d["h0"] if h0 else None, g_hL=d["g_hL"] if g_hL else None,
                            chunk=chunk, want_h0=want_h0)


def _ref(cs, h0=True, g_hL=True):
    return oracle.scan_vjp(cs["k"], cs["dict_idx"], cs["D"].astype(np.float64), cs["Bu"], cs["C"],
                           cs["h0"] if h0 else None, cs["g_y"], cs["g_hL"] if g_hL else None)


@pytest.mark.parametrize("name", list(REDUCED))
def test_states_parity(name):
    cs = _case(name, **REDUCED[name])
    d = _dev(cs)
    print(f"[gpu] pdssm_scan_states {name}", flush=True)
    y, hL, Hs = _gpu_states(d, cs["cfg"].chunk)
    st = oracle.scan_states(cs["k"], cs["dict_idx"], cs["D"].astype(np.float64), cs["Bu"], cs["h0"])
    yr, hLr = oracle.scan(cs["k"], cs["dict_idx"], cs["D"].astype(np.float64), cs["Bu"], cs["C"], cs["h0"])
    assert_within(host(Hs), st, f"{name} states")
    assert_within(host(y), yr, f"{name} y")
    assert_within(host(hL), hLr, f"{name} h_L")


@pytest.mark.parametrize("name", list(REDUCED))
def test_bwd_parity(name):
    cs = _case(name, **REDUCED[name])
    d = _dev(cs)
    chunk = cs["cfg"].chunk
    print(f"[gpu] pdssm_scan_bwd {name} chunk={chunk}", flush=True)
    _, _, Hs = _gpu_states(d, chunk)
    out = _gpu_bwd(d, Hs, chunk)
    g_Bu, g_D, g_h0, g_C = _ref(cs)
    assert_within(host(out["g_Bu"]), g_Bu, f"{name} g_Bu")
    assert_within(host(out["g_D"]), g_D, f"{name} g_D")
    assert_within(host(out["g_h0"]), g_h0, f"{name} g_h0")
    assert_within(host(out["g_C"]), g_C, f"{name} g_C")


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100, 256, 4096])
def test_bwd_chunk_independence(chunk):
    cs = _case("base", B=1, H=2, L=500)
    d = _dev(cs)
    print(f"[gpu] pdssm_scan_bwd base chunk={chunk}", flush=True)
    _, _, Hs = _gpu_states(d, chunk)
    out = _gpu_bwd(d, Hs, chunk)
    g_Bu, g_D, g_h0, g_C = _ref(cs)
    assert_within(host(out["g_Bu"]), g_Bu, f"chunk {chunk} g_Bu")
    assert_within(host(out["g_D"]), g_D, f"chunk {chunk} g_D")
    assert_within(host(out["g_h0"]), g_h0, f"chunk {chunk} g_h0")
    assert_within(host(out["g_C"]), g_C, f"chunk {chunk} g_C")


@pytest.mark.parametrize("N,K", [(1, 1), (5, 3), (12, 7), (16, 16), (17, 4), (40, 9), (32, 16), (64, 32)])
def test_bwd_state_sizes(N, K):
    """State sizes off the power-of-two grid, on both sides of the 16-row
    nibble-path limit, and the time-series and LM-layer state sizes (N = 32
    and 64), with a ragged final chunk."""
    cs = _case("base", B=1, H=2, L=333, N=N, K=K)
    d = _dev(cs)
    g_Bu, g_D, g_h0, g_C = _ref(cs)
    for chunk in (37, 128):
        print(f"[gpu] pdssm_scan_bwd N={N} K={K} chunk={chunk}", flush=True)
        _, _, Hs = _gpu_states(d, chunk)
        out = _gpu_bwd(d, Hs, chunk)
        assert_within(host(out["g_Bu"]), g_Bu, f"N={N} chunk {chunk} g_Bu")
        assert_within(host(out["g_D"]), g_D, f"N={N} chunk {chunk} g_D")
        assert_within(host(out["g_h0"]), g_h0, f"N={N} chunk {chunk} g_h0")
        assert_within(host(out["g_C"]), g_C, f"N={N} chunk {chunk} g_C")


def test_bwd_deterministic():
    cs = _case("impulse", H=4, L=1500)
    d = _dev(cs)
    _, _, Hs = _gpu_states(d, 64)
    a = _gpu_bwd(d, Hs, 64)
    b = _gpu_bwd(d, Hs, 64)
    for n in ("g_Bu", "g_D", "g_h0", "g_C"):
        assert np.array_equal(host(a[n]), host(b[n])), n


def test_bwd_without_h0_and_final_gradient():
    cs = _case("tiny", L=250)
    d = _dev(cs)
    _, _, Hs = _gpu_states(d, 64, h0=False)
    out = _gpu_bwd(d, Hs, 64, h0=False, g_hL=False, want_h0=False)
    g_Bu, g_D, _, g_C = _ref(cs, h0=False, g_hL=False)
    assert "g_h0" not in out
    assert_within(host(out["g_Bu"]), g_Bu, "g_Bu")
    assert_within(host(out["g_D"]), g_D, "g_D")
    assert_within(host(out["g_C"]), g_C, "g_C")


def test_bwd_identity_map_closed_form():
    """P = I, D = 1: dLoss/dBu_s = C * (suffix sum of g_y from s) + g_hL."""
    torch = torch_mod()
    B, H, L, N, K = 1, 2, 777, 8, 3
    rng = np.random.default_rng(5)
    k = rng.integers(0, K, (B, H, L)).astype(np.int32)
    dict_idx = np.tile(np.arange(N, dtype=np.int32), (H, K, 1))
    D = np.ones((B, H, L, N), np.float32)
    Bu = rng.standard_normal((B, H, L, N)).astype(np.float32)
    C = rng.standard_normal((H, N)).astype(np.float32)
    g_y, g_hL = upstream_grads(B, H, L, N, 9)
    d = {n: to_dev(v) for n, v in (("k", k), ("dict_idx", dict_idx), ("D", D), ("Bu", Bu), ("C", C),
                                   ("g_y", g_y), ("g_hL", g_hL))}
    d["h0"] = torch.zeros((B, H, N), device="cuda")
    _, _, Hs = _gpu_states(d, 128)
    out = _gpu_bwd(d, Hs, 128)
    suffix = np.cumsum(g_y[..., ::-1].astype(np.float64), axis=-1)[..., ::-1]
    want = C[None, :, None, :] * suffix[..., None] + g_hL[:, :, None, :]
    assert_within(host(out["g_Bu"]), want, "g_Bu closed form")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_bwd_full_impulse():
    cs = _case("impulse")
    d = _dev(cs)
    chunk = cs["cfg"].chunk
    print(f"[gpu] pdssm_scan_bwd impulse full chunk={chunk}", flush=True)
    _, _, Hs = _gpu_states(d, chunk)
    out = _gpu_bwd(d, Hs, chunk)
    g_Bu, g_D, g_h0, g_C = _ref(cs)
    assert_within(host(out["g_Bu"]), g_Bu, "g_Bu")
    assert_within(host(out["g_D"]), g_D, "g_D")
    assert_within(host(out["g_h0"]), g_h0, "g_h0")
    assert_within(host(out["g_C"]), g_C, "g_C")

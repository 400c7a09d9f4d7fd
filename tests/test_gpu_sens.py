"""Parity of the impulse-sensitivity pass (``pdssm_impulse_sens``, HIP through
the C ABI) with the fp64 oracle (``impulse_sensitivity``).

Selections and diagonals come from the oracle on generated inputs and are fed
to both sides.  Bar: every element of dy_t / du_0 within 1e-4 (1 + |ref|)."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config
from tests._gpu import assert_within, host, lib, proj_dev, to_dev, torch_mod

pytestmark = pytest.mark.gpu

CASES = {
    "impulse": ("impulse", dict(H=3, L=1300)),
    "base": ("base", dict(B=2, H=2, L=700)),
    "tiny": ("tiny", dict(L=250)),
    "bf16_d128": ("timeseries", dict(B=1, H=2, L=600, N=16, K=8)),
    "n5_d32": ("base", dict(B=1, H=2, L=333, N=5, K=3, d=32)),
}

_cache = {}


def _case(key):
    if key not in _cache:
        name, kw = CASES[key]
        inp = generate(get_config(name, **kw))
        k, D, _ = oracle.select(inp.u, inp.W_sel, inp.W_d, inp.b_d, inp.cfg.u_shared)
        D32 = D.astype(np.float32)
        ref = oracle.impulse_sensitivity(k, inp.dict_idx, D32.astype(np.float64), inp.W_d, inp.W_b,
                                         inp.C, inp.h0)
        _cache[key] = (inp, k.astype(np.int32), D32, ref)
    return _cache[key]


def _run(inp, k, D, chunk, h0=True):
    P = lib()
    bf = inp.cfg.dtype == "bf16"
    return P.pdssm_impulse_sens(to_dev(k), to_dev(inp.dict_idx), to_dev(D), proj_dev(inp.W_d, bf),
                                proj_dev(inp.W_b, bf), to_dev(inp.C), to_dev(inp.h0) if h0 else None,
                                chunk=chunk)


@pytest.mark.parametrize("key", list(CASES))
def test_sens_parity(key):
    inp, k, D, ref = _case(key)
    print(f"[gpu] pdssm_impulse_sens {key} chunk={inp.cfg.chunk}", flush=True)
    assert_within(host(_run(inp, k, D, inp.cfg.chunk)), ref, key)


@pytest.mark.parametrize("chunk", [1, 3, 16, 100, 256, 512, 4096])
def test_sens_chunk_independence(chunk):
    inp, k, D, ref = _case("impulse")
    print(f"[gpu] pdssm_impulse_sens impulse chunk={chunk}", flush=True)
    P = lib()
    if chunk > 512:
        with pytest.raises(P.PdssmError) as e:
            _run(inp, k, D, chunk)
        assert e.value.status == P.PDSSM_EUNSUPPORTED
        return
    assert_within(host(_run(inp, k, D, chunk)), ref, f"chunk {chunk}")


def test_sens_without_h0():
    inp, k, D, _ = _case("base")
    ref = oracle.impulse_sensitivity(k, inp.dict_idx, D.astype(np.float64), inp.W_d, inp.W_b, inp.C, None)
    assert_within(host(_run(inp, k, D, inp.cfg.chunk, h0=False)), ref, "h0 = NULL")


def test_sens_deterministic():
    inp, k, D, _ = _case("impulse")
    a = host(_run(inp, k, D, 128))
    b = host(_run(inp, k, D, 128))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,kw", [("base", dict(B=1, H=2, L=64, N=17)),
                                     ("base", dict(B=1, H=2, L=64, d=24)),
                                     ("lm_layer", dict(B=1, H=2, L=64, N=16))])
def test_sens_rejects_unsupported_shapes(name, kw):
    P = lib()
    torch = torch_mod()
    c = get_config(name, **kw)
    B, H, L, N, K, d = c.B, c.H, c.L, c.N, c.K, c.d
    dims = P.make_dims(B, H, L, N, K, d, c.u_shared, False)
    with pytest.raises(P.PdssmError) as e:
        P.impulse_sens_workspace_bytes(dims, 64)
    assert e.value.status == P.PDSSM_EUNSUPPORTED
    del torch


@pytest.mark.slow
def test_sens_full_impulse_sampled_heads():
    """Full impulse shape in the bench's configuration; two heads compared
    element by element with the oracle over all 131072 steps."""
    torch = torch_mod()
    inp = generate(get_config("impulse"))
    k, D, _ = oracle.select(inp.u, inp.W_sel, inp.W_d, inp.b_d, False)
    D32 = D.astype(np.float32)
    print("[gpu] pdssm_impulse_sens impulse full size", flush=True)
    out = _run(inp, k.astype(np.int32), D32, inp.cfg.chunk)
    torch.cuda.synchronize()
    got = host(out)
    for h in (0, 17):
        ref = oracle.impulse_sensitivity(k[:, h:h + 1], inp.dict_idx[h:h + 1], D32[:, h:h + 1].astype(np.float64),
                                         inp.W_d[h:h + 1], inp.W_b[h:h + 1], inp.C[h:h + 1], inp.h0[:, h:h + 1])
        assert_within(got[:, h:h + 1], ref, f"head {h}")

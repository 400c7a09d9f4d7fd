"""Checks of the seeded input generators (CPU only)."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import CONFIGS, GAP, bf16_bits, bf16_round, generate, get_config, top2_margin

SMALL = {
    "tiny": {},
    "base": dict(B=2, H=3, L=700),
    "timeseries": dict(B=2, H=2, L=600),
    "impulse": dict(H=4, L=1500),
    "lm_layer": dict(B=2, H=5, L=300),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_margin_holds_in_oracle_scores(name):
    """Every selection the oracle makes on generated inputs is decided by at
    least GAP (so fp32 and fp64 argmaxes agree)."""
    cfg = get_config(name, **SMALL[name])
    inp = generate(cfg)
    _, _, s = oracle.select(inp.u, inp.W_sel, inp.W_d, inp.b_d, cfg.u_shared)
    assert top2_margin(s).min() >= GAP


@pytest.mark.parametrize("name", list(SMALL))
def test_deterministic_and_thread_independent(name):
    cfg = get_config(name, **SMALL[name])
    a = generate(cfg, threads=1)
    b = generate(cfg, threads=5)
    for f in ("u", "W_sel", "W_d", "W_b", "b_d", "dict_idx", "C", "h0", "Bu"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("name", list(SMALL))
def test_shapes_rules_and_storage(name):
    cfg = get_config(name, **SMALL[name])
    inp = generate(cfg)
    B, H, L, N, K, d = cfg.B, cfg.H, cfg.L, cfg.N, cfg.K, cfg.d
    assert inp.u.shape == ((B, L, d) if cfg.u_shared else (B, H, L, d))
    assert inp.u.dtype == np.float32 and inp.Bu.dtype == np.float32
    assert inp.Bu.shape == (B, H, L, N)
    assert inp.dict_idx.shape == (H, K, N) and inp.dict_idx.dtype == np.int32
    assert inp.dict_idx.min() >= 0 and inp.dict_idx.max() < N
    if cfg.dict_rule == "identity0":
        assert (inp.dict_idx[:, 0] == np.arange(N)).all()
    if cfg.dtype == "bf16":
        for a in (inp.u, inp.W_sel, inp.W_d, inp.W_b):
            assert (a.view(np.uint32) & 0xFFFF == 0).all()
    if cfg.u_rule == "impulse":
        assert np.abs(inp.u[:, :, 0, 0] - 1.0).max() < 0.01
        rest = inp.u.copy()
        rest[:, :, 0, 0] = 0
        assert np.abs(rest).max() < 0.01
    # Bu is W_b u rounded once to fp32
    uu = inp.u.astype(np.float64)
    ref = (np.einsum("blc,hnc->bhln", uu, inp.W_b.astype(np.float64)) if cfg.u_shared
           else np.einsum("bhlc,hnc->bhln", uu, inp.W_b.astype(np.float64)))
    np.testing.assert_allclose(inp.Bu, ref.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e-3], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    r = bf16_round(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0078125) and r[3] == np.float32(1.0078125)
    assert r[4] == -2.5
    assert bf16_bits(np.array([1.0], np.float32))[0] == 0x3F80


def test_config_table():
    assert [CONFIGS[n].seed for n in ("tiny", "base", "timeseries", "impulse", "lm_layer")] == [1, 2, 3, 4, 5]
    c = CONFIGS["impulse"]
    assert (c.B, c.H, c.L, c.N, c.K, c.d, c.chunk) == (1, 32, 131072, 16, 8, 64, 512)
    assert c.state_updates == 67_108_864

"""pdssm_select on the all-heads selection GEMM (u shared by the heads, bf16,
K <= 32, N <= 64 with N a multiple of 4, d a multiple of 64) against the
fp64 oracle's selection.

Bars: k* bit-exact (the generator keeps the top two scores 1e-3 apart; the
tie case below makes them equal on purpose and expects the lowest index);
D within 2e-6; P_idx exactly the dictionary row of k*.  Cases: token counts
that leave a ragged last tile of 256 tokens and a ragged last die class,
one score row, one and two tiles of pre-activation rows, N not a multiple of
32, the LM-layer shape at full size on sampled rows, and agreement with the
per-(rows, head) selection kernel that pdssm_select uses otherwise."""

import os

import numpy as np
import pytest

import oracle
from pdssm_inputs import bf16_round, generate, get_config
from tests._gpu import host, lib, to_dev, torch_mod

pytestmark = pytest.mark.gpu


def _inputs(B, H, L, N, K, d, seed):
    rng = np.random.default_rng(seed)
    u = bf16_round(rng.standard_normal((B, L, d)).astype(np.float32))
    W_sel = bf16_round((rng.standard_normal((H, K, d)) / np.sqrt(d)).astype(np.float32))
    W_d = bf16_round((rng.standard_normal((H, N, d)) / np.sqrt(d)).astype(np.float32))
    b_d = np.full((H, N), 2.0, np.float32) + 0.1 * rng.standard_normal((H, N)).astype(np.float32)
    dic = rng.integers(0, N, size=(H, K, N)).astype(np.int32)
    return u, W_sel, W_d, b_d, dic


def _select(u, W_sel, W_d, b_d, dic, gemm=True):
    torch = torch_mod()
    P = lib()
    old = os.environ.get("PDSSM_GEMM_SEL")
    os.environ["PDSSM_GEMM_SEL"] = "1" if gemm else "0"
    try:
        k, D, Pi = P.pdssm_select(to_dev(u, torch.bfloat16), to_dev(W_sel, torch.bfloat16),
                                  to_dev(W_d, torch.bfloat16), to_dev(b_d), to_dev(dic), want_P=True)
    finally:
        if old is None:
            del os.environ["PDSSM_GEMM_SEL"]
        else:
            os.environ["PDSSM_GEMM_SEL"] = old
    return host(k), host(D), host(Pi)


def _near_ties(s):
    """(b, h, l) whose top two fp32 scores are within 1e-3 (the generator's
    resampling margin; random draws here are not resampled)."""
    s32 = np.sort(s.astype(np.float32), axis=-1)
    return (s32[..., -1] - s32[..., -2]) < 1e-3 if s.shape[-1] > 1 else np.zeros(s.shape[:-1], bool)


CASES = [
    # B, H, L, N, K, d
    (2, 5, 300, 64, 32, 768),     # reduced LM-layer shape: ragged last tile
    (1, 3, 257, 32, 5, 128),      # one tile of pre-activation rows, two channel blocks
    (3, 2, 100, 60, 32, 256),     # N not a multiple of 32
    (2, 1, 513, 64, 1, 384),      # one score row
    (1, 7, 2048, 4, 17, 128),     # smallest N, more tiles than dies
    (2, 3, 200, 64, 32, 64),      # one channel block
    (1, 2, 300, 48, 8, 320),      # an odd number of channel blocks
]


@pytest.mark.parametrize("B,H,L,N,K,d", CASES)
def test_gemm_select_parity(B, H, L, N, K, d):
    u, W_sel, W_d, b_d, dic = _inputs(B, H, L, N, K, d, seed=B * 1000 + L + N)
    print(f"[gpu] gemm select B={B} H={H} L={L} N={N} K={K} d={d}", flush=True)
    k, D, Pi = _select(u, W_sel, W_d, b_d, dic)
    k_ref, D_ref, s = oracle.select(u, W_sel, W_d, b_d, u_shared=True)
    free = ~_near_ties(s)
    assert np.array_equal(k[free], k_ref[free]), f"{int((k[free] != k_ref[free]).sum())} selections differ"
    # where the top two are within the margin, either may be chosen by fp32
    # rounding order: the choice must be one of the maxima within 1e-3
    s32 = s.astype(np.float32)
    chosen = np.take_along_axis(s32, k[..., None].astype(np.int64), axis=-1)[..., 0]
    assert (chosen >= s32.max(axis=-1) - 1e-3).all()
    assert np.abs(D - D_ref).max() <= 2e-6, f"D error {np.abs(D - D_ref).max():.3g}"
    expect = dic[np.arange(H)[None, :, None], k]
    assert np.array_equal(Pi, expect)


def test_gemm_select_ties_lowest_index():
    """Score rows 3, 9 and 20 identical (and the largest): every step must
    choose 3, whichever lanes hold the three rows."""
    B, H, L, N, K, d = 2, 3, 300, 64, 32, 256
    u, W_sel, W_d, b_d, dic = _inputs(B, H, L, N, K, d, seed=99)
    u[..., 0] = np.abs(u[..., 0]) + 1.0
    W_sel = W_sel * 0.01
    W_sel[:, 3] = 0
    W_sel[:, 3, 0] = 4.0
    W_sel[:, 9] = W_sel[:, 3]
    W_sel[:, 20] = W_sel[:, 3]
    W_sel = bf16_round(W_sel)
    print("[gpu] gemm select ties", flush=True)
    k, _, _ = _select(u, W_sel, W_d, b_d, dic)
    assert (k == 3).all()


def test_gemm_select_matches_rows_kernel():
    """The all-heads GEMM and the per-(rows, head) kernel agree on k* exactly
    and on D within 2e-6 (same products, summed in another order)."""
    u, W_sel, W_d, b_d, dic = _inputs(2, 4, 640, 64, 32, 768, seed=5)
    print("[gpu] gemm select vs rows kernel", flush=True)
    kg, Dg, Pg = _select(u, W_sel, W_d, b_d, dic, gemm=True)
    kr, Dr, Pr = _select(u, W_sel, W_d, b_d, dic, gemm=False)
    _, _, s = oracle.select(u, W_sel, W_d, b_d, u_shared=True)
    free = ~_near_ties(s)
    assert np.array_equal(kg[free], kr[free])
    assert np.abs(Dg - Dr).max() <= 2e-6


def test_gemm_select_lm_layer_full_size():
    """The generated LM-layer workload at full size (B=16, H=24, L=2048),
    checked against the oracle on every head of a sample of tokens."""
    torch = torch_mod()
    P = lib()
    cfg = get_config("lm_layer")
    inp = generate(cfg)
    print("[gpu] gemm select lm_layer full size", flush=True)
    k, D = P.pdssm_select(to_dev(inp.u, torch.bfloat16), to_dev(inp.W_sel, torch.bfloat16),
                          to_dev(inp.W_d, torch.bfloat16), to_dev(inp.b_d))
    k, D = host(k), host(D)
    rng = np.random.default_rng(1)
    for b, l0 in [(0, 0), (15, 2047 - 63)] + [(int(x), int(y)) for x, y in
                                               zip(rng.integers(0, 16, 3), rng.integers(0, 2048 - 64, 3))]:
        us = inp.u[b:b + 1, l0:l0 + 64]
        k_ref, D_ref, _ = oracle.select(us, inp.W_sel, inp.W_d, inp.b_d, u_shared=True)
        assert np.array_equal(k[b:b + 1, :, l0:l0 + 64], k_ref), f"batch {b} steps {l0}+: selections differ"
        assert np.abs(D[b:b + 1, :, l0:l0 + 64] - D_ref).max() <= 2e-6

"""Pins of the oracle's forward pass with the drive term formed from the
input (``drive``, ``forward_wb``).

Each check is independent of the oracle's own einsum: a Python double loop on
tiny inputs, a unit weight matrix that copies one input channel into one state
row (closed form), exact superposition in W_b for fixed selections, agreement
with the input generator's own Bu (computed in a separate module, stored in
fp32), and planted mistakes that must fail."""

import numpy as np
import pytest

import oracle
from pdssm_inputs import generate, get_config


def _tiny(seed, B=2, H=3, L=5, N=4, K=3, d=6, shared=False):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, L, d) if shared else (B, H, L, d))
    return dict(
        u=u,
        W_sel=rng.standard_normal((H, K, d)),
        dict_idx=rng.integers(0, N, (H, K, N)),
        W_d=rng.standard_normal((H, N, d)) * 0.5,
        b_d=rng.standard_normal((H, N)),
        W_b=rng.standard_normal((H, N, d)),
        C=rng.standard_normal((H, N)),
        h0=rng.standard_normal((B, H, N)),
        shared=shared,
    )


def _loop_drive(u, W_b, shared):
    B = u.shape[0]
    H, N, d = W_b.shape
    L = u.shape[1] if shared else u.shape[2]
    out = np.zeros((B, H, L, N))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                row = u[b, t] if shared else u[b, h, t]
                for n in range(N):
                    acc = 0.0
                    for c in range(d):
                        acc += float(W_b[h, n, c]) * float(row[c])
                    out[b, h, t, n] = acc
    return out


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_drive_matches_a_double_loop(seed, shared):
    c = _tiny(seed, shared=shared)
    got = oracle.drive(c["u"], c["W_b"], shared)
    assert np.allclose(got, _loop_drive(c["u"], c["W_b"], shared), rtol=1e-13, atol=1e-13)


def test_unit_weight_copies_one_channel_into_one_row():
    """W_b = e_n e_c^T: the drive is channel c of u in state row n, zero elsewhere,
    and the forward pass equals the one given that drive explicitly."""
    c = _tiny(7)
    H, N, d = c["W_b"].shape
    n0, c0 = 2, 4
    W = np.zeros((H, N, d))
    W[:, n0, c0] = 1.0
    Bu = np.zeros(c["u"].shape[:3] + (N,))
    Bu[..., n0] = c["u"][..., c0]
    got = oracle.forward_wb(c["u"], c["W_sel"], c["dict_idx"], c["W_d"], c["b_d"], W, c["C"], c["h0"])
    ref = oracle.forward(c["u"], c["W_sel"], c["dict_idx"], c["W_d"], c["b_d"], Bu, c["C"], c["h0"])
    assert np.array_equal(got["Bu"], Bu)
    assert np.allclose(got["y"], ref["y"], rtol=1e-14, atol=1e-14)
    assert np.allclose(got["h_L"], ref["h_L"], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_superposition_in_the_drive_weights(seed):
    """Selections do not depend on W_b, so y is affine in W_b:
    y(W1 + W2) = y(W1) + y(W2) - y(0)."""
    c = _tiny(seed)
    rng = np.random.default_rng(100 + seed)
    W1, W2 = c["W_b"], rng.standard_normal(c["W_b"].shape)

    def y(W):
        return oracle.forward_wb(c["u"], c["W_sel"], c["dict_idx"], c["W_d"], c["b_d"], W, c["C"],
                                 c["h0"])["y"]

    lhs = y(W1 + W2)
    rhs = y(W1) + y(W2) - y(np.zeros_like(W1))
    assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("name", ["tiny", "impulse"])
def test_agrees_with_the_generators_stored_drive(name):
    """The input generator forms Bu in its own module and stores it in fp32;
    the oracle's fp64 drive must round to it."""
    inp = generate(get_config(name, **({"H": 2, "L": 300} if name == "impulse" else {})))
    got = oracle.drive(inp.u, inp.W_b, inp.cfg.u_shared)
    # within the fp32 rounding of the stored value (half an ulp, 2^-24 relative)
    assert np.all(np.abs(got - inp.Bu) <= 2.0 ** -24 * np.abs(got) + 1e-30)


def test_pins_catch_a_transposed_or_misrouted_drive():
    c = _tiny(3, N=4, d=4)
    loop = _loop_drive(c["u"], c["W_b"], False)
    wrong_t = oracle.drive(c["u"], np.swapaxes(c["W_b"], 1, 2), False)
    assert not np.allclose(wrong_t, loop)
    wrong_head = oracle.drive(c["u"][:, ::-1], c["W_b"], False)
    assert not np.allclose(wrong_head, loop)

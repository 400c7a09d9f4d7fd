"""Pins of the oracle's gradient through the scan (fixed selections).

Each check is independent of ``scan_vjp``'s own recurrence: central finite
differences of the forward ``scan`` (itself pinned in test_oracle_pins.py),
the exact linearity of the loss in (Bu, h0), a closed form for the identity
map with unit diagonal, and planted mistakes that must fail."""

import numpy as np
import pytest

import oracle


def _case(seed, B=2, H=2, L=9, N=5, K=3):
    rng = np.random.default_rng(seed)
    return dict(
        k_star=rng.integers(0, K, (B, H, L)),
        dict_idx=rng.integers(0, N, (H, K, N)),
        D=rng.uniform(0.3, 1.2, (B, H, L, N)),
        Bu=rng.standard_normal((B, H, L, N)),
        C=rng.standard_normal((H, N)),
        h0=rng.standard_normal((B, H, N)),
        g_y=rng.standard_normal((B, H, L)),
        g_hL=rng.standard_normal((B, H, N)),
    )


def _loss(c, **over):
    a = dict(c, **over)
    y, hL = oracle.scan(a["k_star"], a["dict_idx"], a["D"], a["Bu"], a["C"], a["h0"])
    return float((y * a["g_y"]).sum() + (hL * a["g_hL"]).sum())


def _grads(c):
    return oracle.scan_vjp(c["k_star"], c["dict_idx"], c["D"], c["Bu"], c["C"], c["h0"],
                           c["g_y"], c["g_hL"])


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("which", ["Bu", "D", "h0", "C"])
def test_vjp_matches_central_differences(seed, which):
    c = _case(seed)
    g = dict(zip(["Bu", "D", "h0", "C"], _grads(c)))
    rng = np.random.default_rng(100 + seed)
    delta = rng.standard_normal(c[which].shape)
    eps = 1e-6
    fd = (_loss(c, **{which: c[which] + eps * delta}) - _loss(c, **{which: c[which] - eps * delta})) / (2 * eps)
    an = float((g[which] * delta).sum())
    assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (which, fd, an)


@pytest.mark.parametrize("seed", range(3))
def test_loss_is_exactly_linear_in_drive_and_initial_state(seed):
    """For fixed selections and diagonals the loss is a linear form of (Bu, h0)
    plus terms free of them; with C g_y and g_hL as the only sinks, the
    gradients are its coefficients: loss = <g_Bu, Bu> + <g_h0, h0>."""
    c = _case(seed)
    g_Bu, _, g_h0, _ = _grads(c)
    lhs = _loss(c)
    rhs = float((g_Bu * c["Bu"]).sum() + (g_h0 * c["h0"]).sum())
    assert abs(lhs - rhs) <= 1e-12 * (1 + abs(lhs))


def test_identity_map_unit_diagonal_closed_form():
    """P = I, D = 1: h_t = h0 + sum_{s<=t} Bu_s, so dLoss/dBu_s = C * sum_{t>=s}
    g_y[t] + g_hL (a suffix sum), dLoss/dh0 = C * sum_t g_y[t] + g_hL and
    dLoss/dD_t[j] = lam_t[j] h_{t-1}[j]."""
    rng = np.random.default_rng(7)
    B, H, L, N, K = 1, 1, 12, 4, 2
    dict_idx = np.tile(np.arange(N), (H, K, 1))
    c = dict(k_star=rng.integers(0, K, (B, H, L)), dict_idx=dict_idx, D=np.ones((B, H, L, N)),
             Bu=rng.standard_normal((B, H, L, N)), C=rng.standard_normal((H, N)),
             h0=rng.standard_normal((B, H, N)), g_y=rng.standard_normal((B, H, L)),
             g_hL=rng.standard_normal((B, H, N)))
    g_Bu, g_D, g_h0, _ = _grads(c)
    suffix = np.cumsum(c["g_y"][0, 0, ::-1])[::-1]
    want_Bu = c["C"][0][None, :] * suffix[:, None] + c["g_hL"][0, 0][None, :]
    np.testing.assert_allclose(g_Bu[0, 0], want_Bu, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g_h0[0, 0], c["C"][0] * c["g_y"].sum() + c["g_hL"][0, 0], rtol=1e-13)
    states = np.cumsum(c["Bu"][0, 0], axis=0) + c["h0"][0, 0]
    prev = np.vstack([c["h0"][0, 0][None], states[:-1]])
    np.testing.assert_allclose(g_D[0, 0], want_Bu * prev, rtol=1e-12, atol=1e-12)


def test_states_match_scan_outputs():
    c = _case(11)
    st = oracle.scan_states(c["k_star"], c["dict_idx"], c["D"], c["Bu"], c["h0"])
    y, hL = oracle.scan(c["k_star"], c["dict_idx"], c["D"], c["Bu"], c["C"], c["h0"])
    np.testing.assert_allclose(st[:, :, -1], hL, rtol=1e-14)
    np.testing.assert_allclose((st * c["C"][None, :, None, :]).sum(-1), y, rtol=1e-12, atol=1e-12)


def _vjp_untransposed(k_star, dict_idx, D, Bu, C, h0, g_y, g_hL):
    """A planted mistake: propagate the adjoint with A_t instead of A_t^T."""
    B, H, L = k_star.shape
    N = dict_idx.shape[-1]
    lam = np.array(g_hL, dtype=float)
    g_Bu = np.zeros((B, H, L, N))
    for t in range(L - 1, -1, -1):
        lam = lam + C[None] * g_y[:, :, t, None]
        g_Bu[:, :, t] = lam
        A = oracle.transition_matrix(dict_idx[np.arange(H)[None, :], k_star[:, :, t]], D[:, :, t])
        lam = np.matmul(A, lam[..., None])[..., 0]
    return g_Bu


def test_pins_catch_an_untransposed_adjoint():
    c = _case(3, N=6)
    g_Bu = _vjp_untransposed(c["k_star"], c["dict_idx"], c["D"], c["Bu"], c["C"], c["h0"], c["g_y"], c["g_hL"])
    rhs = float((g_Bu * c["Bu"]).sum())
    g_h0 = _grads(c)[2]
    lhs = _loss(c) - float((g_h0 * c["h0"]).sum())
    assert abs(lhs - rhs) > 1e-6 * (1 + abs(lhs))

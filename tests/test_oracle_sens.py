"""Pins of the oracle's impulse sensitivity dy_t / du_0 (fixed selections).

Each check is independent of ``impulse_sensitivity``'s own tangent
recurrence: central finite differences of the whole forward pass
(``forward_wb``, which re-selects and recomputes D and Bu from the perturbed
input), the forward-mode / reverse-mode identity against ``scan_vjp``, a
closed form for the identity map with a constant diagonal, and a planted
mistake that must fail."""

import numpy as np
import pytest

import oracle


def _case(seed, B=1, H=2, L=7, N=4, K=3, d=5):
    rng = np.random.default_rng(seed)
    return dict(
        u=rng.standard_normal((B, H, L, d)),
        W_sel=rng.standard_normal((H, K, d)),
        dict_idx=rng.integers(0, N, (H, K, N)),
        W_d=rng.standard_normal((H, N, d)) * 0.7,
        b_d=rng.standard_normal((H, N)) * 0.5,
        W_b=rng.standard_normal((H, N, d)),
        C=rng.standard_normal((H, N)),
        h0=rng.standard_normal((B, H, N)),
    )


def _fwd(c, u):
    return oracle.forward_wb(u, c["W_sel"], c["dict_idx"], c["W_d"], c["b_d"], c["W_b"], c["C"], c["h0"])


def _sens(c):
    f = _fwd(c, c["u"])
    return f, oracle.impulse_sensitivity(f["k_star"], c["dict_idx"], f["D"], c["W_d"], c["W_b"], c["C"],
                                         c["h0"])


@pytest.mark.parametrize("seed", range(4))
def test_matches_central_differences_of_the_forward_pass(seed):
    c = _case(seed)
    f0, got = _sens(c)
    eps = 1e-6
    d = c["u"].shape[-1]
    for ch in range(d):
        up, dn = c["u"].copy(), c["u"].copy()
        up[:, :, 0, ch] += eps
        dn[:, :, 0, ch] -= eps
        fu, fd = _fwd(c, up), _fwd(c, dn)
        # the perturbation must not change a selection (derivative of a fixed choice)
        assert np.array_equal(fu["k_star"], f0["k_star"]) and np.array_equal(fd["k_star"], f0["k_star"])
        fd_est = (fu["y"] - fd["y"]) / (2 * eps)
        assert np.allclose(got[..., ch], fd_est, rtol=1e-6, atol=1e-8), ch


@pytest.mark.parametrize("seed", range(3))
def test_forward_mode_agrees_with_reverse_mode(seed):
    """<g_y, dy/du_0[c]> equals the gradient of <g_y, y> with respect to u_0[c]
    assembled from the adjoint: dBu_0 . W_b[:, c] + sum_j dD_0[j] D_0[j] (1 - D_0[j]) W_d[j, c]."""
    c = _case(seed)
    f, sens = _sens(c)
    rng = np.random.default_rng(50 + seed)
    g_y = rng.standard_normal(f["y"].shape)
    Bu = oracle.drive(c["u"], c["W_b"])
    g_Bu, g_D, _, _ = oracle.scan_vjp(f["k_star"], c["dict_idx"], f["D"], Bu, c["C"], c["h0"], g_y)
    D0 = f["D"][:, :, 0]
    lhs = np.einsum("bhl,bhlc->bhc", g_y, sens)
    rhs = (np.einsum("bhn,hnc->bhc", g_Bu[:, :, 0], c["W_b"])
           + np.einsum("bhn,hnc->bhc", g_D[:, :, 0] * D0 * (1 - D0), c["W_d"]))
    assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_identity_map_constant_diagonal_closed_form():
    """P = I and D_t = delta: V_t = delta^t J with J = W_b + diag(delta (1 - delta) h0) W_d."""
    rng = np.random.default_rng(9)
    B, H, L, N, K, d = 1, 2, 10, 3, 2, 4
    dict_idx = np.tile(np.arange(N), (H, K, 1))
    k = rng.integers(0, K, (B, H, L))
    delta = 0.8
    D = np.full((B, H, L, N), delta)
    W_d, W_b = rng.standard_normal((H, N, d)), rng.standard_normal((H, N, d))
    C, h0 = rng.standard_normal((H, N)), rng.standard_normal((B, H, N))
    got = oracle.impulse_sensitivity(k, dict_idx, D, W_d, W_b, C, h0)
    for h in range(H):
        J = W_b[h] + (delta * (1 - delta) * h0[0, h])[:, None] * W_d[h]
        for t in range(L):
            assert np.allclose(got[0, h, t], delta ** t * (C[h] @ J), rtol=1e-13, atol=1e-13)


def test_pin_catches_a_double_counted_first_step():
    """Applying A_0 to the step-0 tangent again (off by one step) must fail
    the finite-difference pin."""
    c = _case(1)
    f, good = _sens(c)
    idx0 = c["dict_idx"][np.arange(2), f["k_star"][0, :, 0]]
    bad = np.empty_like(good)
    for h in range(2):
        A0 = oracle.transition_matrix(idx0[h], f["D"][0, h, 0])
        # the wrong tangent starts one transition too late: A_0 applied to J
        J = c["W_b"][h] + oracle.transition_matrix(idx0[h], f["D"][0, h, 0] * (1 - f["D"][0, h, 0])
                                                   * c["h0"][0, h]) @ c["W_d"][h]
        V = A0 @ J
        bad[0, h, 0] = c["C"][h] @ V
        for t in range(1, good.shape[2]):
            V = oracle.transition_matrix(c["dict_idx"][h, f["k_star"][0, h, t]], f["D"][0, h, t]) @ V
            bad[0, h, t] = c["C"][h] @ V
    assert not np.allclose(bad, good, rtol=1e-6, atol=1e-8)

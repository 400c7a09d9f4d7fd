"""Pins of the oracle's several-outputs-per-head scan (``scan_multi``,
``forward_wb_multi``): y[b,h,t,o] = C[h,o,:] . h_t.

Independent of ``scan_multi``'s own einsum over the saved states: Python
loops with an explicit scatter-add on tiny inputs, the single-output scan
(which computes y inside its own step loop) for every row of C, the fused
forward with the drive formed from u, and a planted mistake that must fail."""

import numpy as np
import pytest

import oracle


def _case(seed, B=2, H=3, L=9, N=5, K=3, P=3):
    rng = np.random.default_rng(seed)
    return dict(
        k=rng.integers(0, K, (B, H, L)),
        dic=rng.integers(0, N, (H, K, N)),
        D=rng.uniform(0.3, 1.1, (B, H, L, N)),
        Bu=rng.standard_normal((B, H, L, N)),
        C=rng.standard_normal((H, P, N)),
        h0=rng.standard_normal((B, H, N)),
    )


def _loops(c):
    k, dic, D, Bu, C, h0 = c["k"], c["dic"], c["D"], c["Bu"], c["C"], c["h0"]
    B, H, L = k.shape
    P, N = C.shape[1], C.shape[2]
    y = np.zeros((B, H, L, P))
    hL = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            x = [float(v) for v in h0[b, h]]
            for t in range(L):
                nx = [float(v) for v in Bu[b, h, t]]
                for j in range(N):
                    nx[dic[h, k[b, h, t], j]] += float(D[b, h, t, j]) * x[j]
                x = nx
                for o in range(P):
                    y[b, h, t, o] = sum(float(C[h, o, n]) * x[n] for n in range(N))
            hL[b, h] = x
    return y, hL


@pytest.mark.parametrize("seed", range(3))
def test_matches_loops(seed):
    c = _case(seed)
    y, hL = oracle.scan_multi(c["k"], c["dic"], c["D"], c["Bu"], c["C"], c["h0"])
    yl, hl = _loops(c)
    assert np.allclose(y, yl, rtol=1e-13, atol=1e-13)
    assert np.allclose(hL, hl, rtol=1e-13, atol=1e-13)


def test_every_row_is_the_single_output_scan():
    c = _case(5, L=40, N=7, P=4)
    y, hL = oracle.scan_multi(c["k"], c["dic"], c["D"], c["Bu"], c["C"], c["h0"])
    for o in range(c["C"].shape[1]):
        ys, hs = oracle.scan(c["k"], c["dic"], c["D"], c["Bu"], c["C"][:, o], c["h0"])
        assert np.allclose(y[..., o], ys, rtol=1e-13, atol=1e-13), o
        assert np.array_equal(hL, hs)


def test_forward_wb_multi_is_forward_wb_per_row():
    rng = np.random.default_rng(6)
    B, H, L, N, K, d, P = 1, 2, 30, 6, 4, 8, 3
    u = rng.standard_normal((B, H, L, d))
    W_sel, W_d, W_b = (rng.standard_normal((H, K, d)), rng.standard_normal((H, N, d)) * 0.5,
                       rng.standard_normal((H, N, d)))
    b_d = rng.standard_normal((H, N))
    dic = rng.integers(0, N, (H, K, N))
    C = rng.standard_normal((H, P, N))
    h0 = rng.standard_normal((B, H, N))
    m = oracle.forward_wb_multi(u, W_sel, dic, W_d, b_d, W_b, C, h0)
    for o in range(P):
        f = oracle.forward_wb(u, W_sel, dic, W_d, b_d, W_b, C[:, o], h0)
        assert np.array_equal(f["k_star"], m["k_star"]) and np.array_equal(f["Bu"], m["Bu"])
        assert np.allclose(f["y"], m["y"][..., o], rtol=1e-13, atol=1e-13)


def test_pin_catches_a_transposed_output_matrix():
    """Reading C as [H,N,n_out] (square here, so the shapes agree) must fail
    the per-row pin."""
    c = _case(7, N=4, P=4)
    bad, _ = oracle.scan_multi(c["k"], c["dic"], c["D"], c["Bu"], np.swapaxes(c["C"], 1, 2), c["h0"])
    ys, _ = oracle.scan(c["k"], c["dic"], c["D"], c["Bu"], c["C"][:, 1], c["h0"])
    assert not np.allclose(bad[..., 1], ys, rtol=1e-6, atol=1e-8)

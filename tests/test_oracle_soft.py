"""Pins of the oracle's soft-selection comparison path (``soft_select``,
``scan_pidx``, ``dict_hardmax``).

Independent of the oracle's own vectorised code: Python loops on tiny
inputs, the reduction to the hard-selection path when K = 1 and when one
score dominates (the hard selection is the limit of the soft one), the
softmax's invariants, the per-step scan against the dictionary scan when the
per-step maps come from a dictionary, and planted mistakes that must fail."""

import math

import numpy as np
import pytest

import oracle


def _tiny(seed, B=1, H=2, L=6, N=4, K=3, d=5):
    rng = np.random.default_rng(seed)
    return dict(
        u=rng.standard_normal((B, H, L, d)),
        W_sel=rng.standard_normal((H, K, d)),
        M=rng.standard_normal((H, K, N, N)),
        W_d=rng.standard_normal((H, N, d)) * 0.5,
        b_d=rng.standard_normal((H, N)),
        Bu=rng.standard_normal((B, H, L, N)),
        C=rng.standard_normal((H, N)),
        h0=rng.standard_normal((B, H, N)),
    )


def _loop_soft(c):
    u, Ws, M, Wd, bd = c["u"], c["W_sel"], c["M"], c["W_d"], c["b_d"]
    B, H, L, d = u.shape
    K, N = M.shape[1], M.shape[2]
    P = np.zeros((B, H, L, N), dtype=int)
    Dv = np.zeros((B, H, L, N))
    Mt = np.zeros((B, H, L, N, N))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                s = [sum(float(Ws[h, k, q]) * float(u[b, h, t, q]) for q in range(d)) for k in range(K)]
                mx = max(s)
                e = [math.exp(v - mx) for v in s]
                a = [v / sum(e) for v in e]
                for i in range(N):
                    for j in range(N):
                        Mt[b, h, t, i, j] = sum(a[k] * float(M[h, k, i, j]) for k in range(K))
                for j in range(N):
                    best = 0
                    for i in range(1, N):
                        if Mt[b, h, t, i, j] > Mt[b, h, t, best, j]:
                            best = i
                    P[b, h, t, j] = best
                    z = sum(float(Wd[h, j, q]) * float(u[b, h, t, q]) for q in range(d)) + float(bd[h, j])
                    Dv[b, h, t, j] = 1.0 / (1.0 + math.exp(-z))
    return Mt, P, Dv


@pytest.mark.parametrize("seed", range(3))
def test_soft_select_matches_loops(seed):
    c = _tiny(seed)
    got = oracle.soft_select(c["u"], c["W_sel"], c["M"], c["W_d"], c["b_d"])
    Mt, P, Dv = _loop_soft(c)
    assert np.allclose(got["M_t"], Mt, rtol=1e-13, atol=1e-13)
    assert np.array_equal(got["P_idx"], P)
    assert np.allclose(got["D"], Dv, rtol=1e-13, atol=1e-13)


def test_softmax_invariants():
    c = _tiny(4, K=5)
    a = oracle.soft_select(c["u"], c["W_sel"], c["M"], c["W_d"], c["b_d"])["alpha"]
    s = oracle.scores(c["u"], c["W_sel"], False)
    assert np.all(a >= 0) and np.allclose(a.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(np.log(a[..., 1] / a[..., 0]), s[..., 1] - s[..., 0], rtol=1e-12, atol=1e-12)


def test_single_matrix_reduces_to_the_hard_path():
    """K = 1: alpha = 1, every M_t is M[h,0], so the soft path is the hard path
    with the column-hardmax dictionary and k* = 0."""
    c = _tiny(5, K=1)
    got = oracle.soft_select(c["u"], c["W_sel"], c["M"], c["W_d"], c["b_d"])
    dic = oracle.dict_hardmax(c["M"])
    y1, h1 = oracle.scan_pidx(got["P_idx"], got["D"], c["Bu"], c["C"], c["h0"])
    k = np.zeros(c["u"].shape[:3], dtype=int)
    y2, h2 = oracle.scan(k, dic, got["D"], c["Bu"], c["C"], c["h0"])
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_a_dominant_score_gives_the_hard_selection():
    """Scores far apart make alpha one-hot in fp64, so M_t = M[h,k*] and the
    soft path's maps are the dictionary rows of the hard path at k*."""
    c = _tiny(6, K=4, N=5, L=8)
    W = c["W_sel"] * 400.0
    got = oracle.soft_select(c["u"], W, c["M"], c["W_d"], c["b_d"])
    k, _, _ = oracle.select(c["u"], W, c["W_d"], c["b_d"])
    s = np.sort(oracle.scores(c["u"], W, False), axis=-1)
    far = s[..., -1] - s[..., -2] > 60                   # exp(-60): alpha one-hot to 1e-26
    assert far.mean() > 0.8
    dic = oracle.dict_hardmax(c["M"])
    H = c["M"].shape[0]
    want = dic[np.arange(H)[None, :, None], k]
    assert np.array_equal(got["P_idx"][far], want[far])


def test_scan_pidx_equals_the_dictionary_scan_on_dictionary_maps():
    rng = np.random.default_rng(7)
    B, H, L, N, K = 2, 3, 20, 6, 4
    dic = rng.integers(0, N, (H, K, N))
    k = rng.integers(0, K, (B, H, L))
    D = rng.uniform(0.2, 1.1, (B, H, L, N))
    Bu = rng.standard_normal((B, H, L, N))
    C = rng.standard_normal((H, N))
    h0 = rng.standard_normal((B, H, N))
    P = dic[np.arange(H)[None, :, None], k]
    y1, h1 = oracle.scan_pidx(P, D, Bu, C, h0)
    y2, h2 = oracle.scan(k, dic, D, Bu, C, h0)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_dict_hardmax_ties_go_to_the_lowest_row_and_gap_is_zero_on_ties():
    M = np.zeros((1, 1, 3, 3))
    M[0, 0, :, 0] = [1.0, 2.0, 2.0]      # tie between rows 1 and 2
    M[0, 0, :, 1] = [5.0, 1.0, 0.0]
    M[0, 0, :, 2] = [0.0, 0.0, 3.0]
    assert list(oracle.dict_hardmax(M)[0, 0]) == [1, 0, 2]
    u = np.zeros((1, 1, 1, 2))
    got = oracle.soft_select(u, np.zeros((1, 1, 2)), M, np.zeros((1, 3, 2)), np.zeros((1, 3)))
    assert list(got["gap"][0, 0, 0]) == [0.0, 4.0, 3.0]


def test_pins_catch_a_row_hardmax_and_a_transposed_mixture():
    c = _tiny(8, N=5)
    _, P, _ = _loop_soft(c)
    got = oracle.soft_select(c["u"], c["W_sel"], c["M"], c["W_d"], c["b_d"])
    row_wise = np.argmax(got["M_t"], axis=-1)
    assert not np.array_equal(row_wise, P)
    tr = oracle.soft_select(c["u"], c["W_sel"], np.swapaxes(c["M"], -1, -2), c["W_d"], c["b_d"])
    assert not np.array_equal(tr["P_idx"], P)

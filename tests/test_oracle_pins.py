"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: a hand-worked example, a closed
form, a library routine, an integer simulation of an automaton, brute force in
exact rational arithmetic, or an algebraic identity.  Planted-mistake checks
(``test_pins_catch_*``) confirm that plausible slips in the oracle's arithmetic
would fail these pins.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import pdssm_oracle as po

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _one_seq(x):
    """[L, ...] -> [1, 1, L, ...]"""
    return np.asarray(x)[None, None]


# --------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_worked_scan.json)
# --------------------------------------------------------------------------

def _hand_scan(scan_fn=oracle.scan):
    g = _load("hand_worked_scan.json")
    dic = np.array(g["dict"], dtype=np.int32)[None]           # [1,K,N]
    ks = _one_seq(np.array(g["k_star"], dtype=np.int32))
    D = _one_seq(np.array(g["D"]))
    Bu = _one_seq(np.array(g["Bu"]))
    C = np.array(g["C"])[None]
    h0 = np.array(g["h0"])[None, None]
    return g, scan_fn(ks, dic, D, Bu, C, h0), (ks, dic, D, Bu, C, h0)


def test_hand_worked_scan_exact():
    g, (y, hL), (ks, dic, D, Bu, C, h0) = _hand_scan()
    assert y[0, 0].tolist() == g["expected_y"]
    assert hL[0, 0].tolist() == g["expected_h_L"]
    for t, state in enumerate(g["expected_states"]):      # every prefix's final state
        _, hx = oracle.scan(ks[..., :t + 1], dic, D[:, :, :t + 1], Bu[:, :, :t + 1], C, h0)
        assert hx[0, 0].tolist() == state


# --------------------------------------------------------------------------
# F1: brute force in exact rational arithmetic, differently associated
# --------------------------------------------------------------------------

def _frac_matrix(idx, dvals):
    N = len(idx)
    A = [[Fraction(0)] * N for _ in range(N)]
    for j in range(N):
        A[idx[j]][j] = Fraction(dvals[j])
    return A


def _mm(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][k] * B[k][j] for k in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _mv(A, x):
    return [sum((A[i][j] * x[j] for j in range(len(x))), Fraction(0)) for i in range(len(A))]


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_products_exact(seed):
    """h_L = (A_{L-1}...A_0) h0 + sum_t (A_{L-1}...A_{t+1}) Bu_t and
    y_t = C h_t, evaluated with explicit rational matrix products."""
    rng = np.random.default_rng(100 + seed)
    N, K, L = int(rng.integers(2, 5)), int(rng.integers(1, 4)), int(rng.integers(1, 13))
    dic = rng.integers(0, N, size=(1, K, N)).astype(np.int32)
    ks = rng.integers(0, K, size=(1, 1, L)).astype(np.int32)
    D = rng.integers(1, 5, size=(1, 1, L, N)) / 4.0           # dyadic, exact in fp64
    Bu = rng.integers(-4, 5, size=(1, 1, L, N)).astype(np.float64)
    C = rng.integers(-3, 4, size=(1, N)).astype(np.float64)
    h0 = rng.integers(-4, 5, size=(1, 1, N)).astype(np.float64)
    y, hL = oracle.scan(ks, dic, D, Bu, C, h0)

    A = [_frac_matrix(dic[0, ks[0, 0, t]].tolist(), D[0, 0, t].tolist()) for t in range(L)]
    eye = [[Fraction(int(i == j)) for j in range(N)] for i in range(N)]

    def prod(lo, hi):        # A_{hi-1} ... A_{lo}
        P = eye
        for t in range(lo, hi):
            P = _mm(A[t], P)
        return P

    for t in range(L):
        h = _mv(prod(0, t + 1), [Fraction(v) for v in h0[0, 0]])
        for s in range(t + 1):
            term = _mv(prod(s + 1, t + 1), [Fraction(v) for v in Bu[0, 0, s]])
            h = [a + b for a, b in zip(h, term)]
        yt = sum((Fraction(C[0, i]) * h[i] for i in range(N)), Fraction(0))
        assert y[0, 0, t] == float(yt)
        if t == L - 1:
            assert hL[0, 0].tolist() == [float(v) for v in h]


# --------------------------------------------------------------------------
# F2: closure of PD maps; O(N) apply / compose against dense products
# --------------------------------------------------------------------------

@pytest.mark.parametrize("span", [1, 2, 5, 17, 64])
def test_closure_and_compose(span):
    rng = np.random.default_rng(span)
    N = 12
    idxs = rng.integers(0, N, size=(span, N))
    scs = rng.uniform(0.1, 1.0, size=(span, N))
    dense = np.eye(N)
    comp = (np.arange(N), np.ones(N))
    for t in range(span):
        A = oracle.transition_matrix(idxs[t], scs[t])
        dense = A @ dense
        comp = oracle.pd_compose((idxs[t], scs[t]), comp)
    nz = dense != 0
    assert (nz.sum(axis=0) == 1).all(), "product must keep one nonzero per column"
    assert (np.argmax(nz, axis=0) == comp[0]).all()
    np.testing.assert_allclose(dense[comp[0], np.arange(N)], comp[1], rtol=1e-15, atol=0)
    x = rng.standard_normal(N)
    b = rng.standard_normal(N)
    np.testing.assert_allclose(oracle.pd_apply(comp[0], comp[1], x, b), dense @ x + b,
                               rtol=1e-13, atol=1e-13)


def test_transition_matrix_orientation():
    """Column j carries D[j] in row idx[j]: A e_j = D[j] e_{idx[j]}."""
    idx = np.array([2, 0, 0])
    d = np.array([0.5, 0.25, 2.0])
    A = oracle.transition_matrix(idx, d)
    for j in range(3):
        e = np.zeros(3)
        e[j] = 1
        expect = np.zeros(3)
        expect[idx[j]] = d[j]
        assert (A @ e).tolist() == expect.tolist()


# --------------------------------------------------------------------------
# F3: chunk-size independence of the three-phase evaluation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 2, 3, 7, 16, 40])
def test_three_phase_matches_sequential(chunk):
    rng = np.random.default_rng(7)
    B, H, L, N, K = 2, 3, 40, 6, 4
    dic = rng.integers(0, N, size=(H, K, N)).astype(np.int32)
    ks = rng.integers(0, K, size=(B, H, L)).astype(np.int32)
    D = rng.uniform(0.3, 1.0, size=(B, H, L, N))
    Bu = rng.standard_normal((B, H, L, N))
    C = rng.standard_normal((H, N))
    h0 = rng.standard_normal((B, H, N))
    y, hL = oracle.scan(ks, dic, D, Bu, C, h0)
    y3, hL3 = oracle.three_phase(ks, dic, D, Bu, C, h0, chunk=chunk)
    np.testing.assert_allclose(y3, y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hL3, hL, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# F4: P = I, D = 1 reduces to a prefix sum
# --------------------------------------------------------------------------

def test_identity_unit_diagonal_is_prefix_sum():
    rng = np.random.default_rng(4)
    B, H, L, N = 2, 2, 300, 5
    dic = np.broadcast_to(np.arange(N), (H, 1, N)).astype(np.int32)
    ks = np.zeros((B, H, L), dtype=np.int32)
    D = np.ones((B, H, L, N))
    Bu = rng.standard_normal((B, H, L, N))
    C = rng.standard_normal((H, N))
    h0 = rng.standard_normal((B, H, N))
    y, hL = oracle.scan(ks, dic, D, Bu, C, h0)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                exact = math.fsum([h0[b, h, i], *Bu[b, h, :, i]])
                assert abs(hL[b, h, i] - exact) <= 1e-12 * (1 + abs(exact))
    states = h0[:, :, None, :] + np.cumsum(Bu, axis=2)
    np.testing.assert_allclose(y, (states * C[None, :, None, :]).sum(-1), rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------
# F5: closed-form impulse responses
# --------------------------------------------------------------------------

def test_single_step_scatter_is_bincount():
    rng = np.random.default_rng(5)
    N = 9
    for _ in range(20):
        idx = rng.integers(0, N, size=N)
        d = rng.uniform(0.1, 1.0, size=N)
        h0 = rng.standard_normal(N)
        bu = rng.standard_normal(N)
        C = rng.standard_normal(N)
        _, hL = oracle.scan(np.zeros((1, 1, 1), np.int32), idx[None, None], d[None, None, None],
                            bu[None, None, None], C[None], h0[None, None])
        expect = np.bincount(idx, weights=d * h0, minlength=N) + bu
        np.testing.assert_allclose(hL[0, 0], expect, rtol=1e-15, atol=1e-15)


def test_cyclic_shift_impulse_closed_form():
    """idx[j] = (j+1) mod N, constant D = diag(d), Bu_0 = b, Bu_{t>0} = 0, h0 = 0:
    h_t[(j+t) mod N] = prod_{m<t} d[(j+m) mod N] * b[j]."""
    rng = np.random.default_rng(55)
    N, L = 7, 30
    idx = (np.arange(N) + 1) % N
    d = rng.uniform(0.5, 1.0, size=N)
    b = rng.standard_normal(N)
    C = rng.standard_normal(N)
    Bu = np.zeros((1, 1, L, N))
    Bu[0, 0, 0] = b
    y, _ = oracle.scan(np.zeros((1, 1, L), np.int32), idx[None, None],
                       np.broadcast_to(d, (1, 1, L, N)), Bu, C[None])
    for t in range(L):
        expect = 0.0
        for j in range(N):
            path = math.prod(d[(j + m) % N] for m in range(t))
            expect += C[(j + t) % N] * path * b[j]
        assert abs(y[0, 0, t] - expect) <= 1e-13 * (1 + abs(expect))
    # scalar decay: every path product is d^t
    y2, _ = oracle.scan(np.zeros((1, 1, L), np.int32), idx[None, None],
                        np.full((1, 1, L, N), 0.75), Bu, C[None])
    for t in range(L):
        expect = sum(C[(j + t) % N] * 0.75 ** t * b[j] for j in range(N))
        assert abs(y2[0, 0, t] - expect) <= 1e-13 * (1 + abs(expect))


# --------------------------------------------------------------------------
# F6: automata (Proposition 1) through selection and scan
# --------------------------------------------------------------------------

def fsa_inputs(delta, symbols, start, d=8):
    """Encode a DFA: K = #symbols, dictionary row k is delta[k]; u_t is the
    one-hot symbol in the first K of d channels; W_sel = 4 [I_K | 0] (margin
    4); W_d = 0 and b_d = 40 (sigmoid(40) rounds to 1 in fp32 and fp64);
    Bu = 0; h0 = e_start."""
    delta = np.asarray(delta, dtype=np.int32)
    K, N = delta.shape
    L = len(symbols)
    u = np.zeros((1, 1, L, d))
    u[0, 0, np.arange(L), symbols] = 1.0
    W_sel = np.zeros((1, K, d))
    W_sel[0, :, :K] = 4.0 * np.eye(K)
    W_d = np.zeros((1, N, d))
    b_d = np.full((1, N), 40.0)
    Bu = np.zeros((1, 1, L, N))
    h0 = np.zeros((1, 1, N))
    h0[0, 0, start] = 1.0
    return u, W_sel, delta[None], W_d, b_d, Bu, h0


def _simulate(delta, symbols, start):
    q, out = start, []
    for s in symbols:
        q = delta[s][q]
        out.append(q)
    return out


def test_sigmoid_40_is_one():
    assert oracle.sigmoid(40.0) == 1.0
    assert np.float32(1.0) / (np.float32(1.0) + np.exp(np.float32(-40.0))) == np.float32(1.0)


@pytest.mark.parametrize("name", ["parity", "mod3_count", "cycle5"])
def test_fsa_fixture_automata(name):
    a = _load("automata.json")["automata"][name]
    N = a["N"]
    C = np.arange(1, N + 1, dtype=np.float64)[None] * 10.0
    for case in a["cases"]:
        sy = case["symbols"]
        u, W_sel, dic, W_d, b_d, Bu, h0 = fsa_inputs(a["delta"], sy, a["start"])
        out = oracle.forward(u, W_sel, dic, W_d, b_d, Bu, C, h0)
        assert out["k_star"][0, 0].tolist() == sy
        qs = _simulate(a["delta"], sy, a["start"])
        assert qs[-1] == case["final"]
        assert out["y"][0, 0].tolist() == [C[0, q] for q in qs]
        onehot = np.zeros(N)
        onehot[case["final"]] = 1.0
        assert out["h_L"][0, 0].tolist() == onehot.tolist()


@pytest.mark.parametrize("seed", range(4))
def test_fsa_random_dfa(seed):
    """Random (non-permutation) automata: the state stays one-hot and follows
    the integer simulation."""
    rng = np.random.default_rng(900 + seed)
    N, K, L = int(rng.integers(3, 9)), int(rng.integers(2, 6)), 60
    delta = rng.integers(0, N, size=(K, N))
    sy = rng.integers(0, K, size=L).tolist()
    start = int(rng.integers(0, N))
    u, W_sel, dic, W_d, b_d, Bu, h0 = fsa_inputs(delta, sy, start)
    C = rng.standard_normal((1, N))
    out = oracle.forward(u, W_sel, dic, W_d, b_d, Bu, C, h0)
    qs = _simulate(delta.tolist(), sy, start)
    assert out["y"][0, 0].tolist() == [C[0, q] for q in qs]


# --------------------------------------------------------------------------
# F7, F8: linearity and resume
# --------------------------------------------------------------------------

def _rand_scan_inputs(seed, B=2, H=3, L=50, N=7, K=5):
    rng = np.random.default_rng(seed)
    return dict(
        k_star=rng.integers(0, K, size=(B, H, L)).astype(np.int32),
        dict_idx=rng.integers(0, N, size=(H, K, N)).astype(np.int32),
        D=rng.uniform(0.2, 1.0, size=(B, H, L, N)),
        Bu=rng.standard_normal((B, H, L, N)),
        C=rng.standard_normal((H, N)),
        h0=rng.standard_normal((B, H, N)),
    ), rng


def test_linearity():
    a, rng = _rand_scan_inputs(71)
    Bu2 = rng.standard_normal(a["Bu"].shape)
    y12, h12 = oracle.scan(a["k_star"], a["dict_idx"], a["D"], a["Bu"] + Bu2, a["C"], a["h0"])
    y1, h1 = oracle.scan(a["k_star"], a["dict_idx"], a["D"], a["Bu"], a["C"], a["h0"])
    y2, h2 = oracle.scan(a["k_star"], a["dict_idx"], a["D"], Bu2, a["C"], None)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h12, h1 + h2, rtol=1e-12, atol=1e-12)


def test_resume_is_bit_identical():
    a, _ = _rand_scan_inputs(81)
    y, hL = oracle.scan(**a)
    L1 = 23
    part = {k: (v[:, :, :L1] if k in ("k_star", "D", "Bu") else v) for k, v in a.items()}
    ya, ha = oracle.scan(**part)
    rest = {k: (v[:, :, L1:] if k in ("k_star", "D", "Bu") else v) for k, v in a.items()}
    rest["h0"] = ha
    yb, hb = oracle.scan(**rest)
    assert np.array_equal(np.concatenate([ya, yb], axis=2), y)
    assert np.array_equal(hb, hL)


# --------------------------------------------------------------------------
# F9: argmax ties go to the lowest index
# --------------------------------------------------------------------------

def test_argmax_ties_lowest_index():
    rng = np.random.default_rng(9)
    H, K, d, L = 2, 6, 8, 40
    u = rng.standard_normal((1, H, L, d))
    W = rng.standard_normal((H, K, d)) * 0.01
    k1, k2 = 1, 4
    big = np.zeros(d)
    big[0] = 5.0
    W[:, k1] = big
    W[:, k2] = big                      # identical rows: identical scores
    u[..., 0] = np.abs(u[..., 0]) + 1.0  # make those scores the maximum
    k_star, _, s = oracle.select(u, W, np.zeros((H, 3, d)), np.zeros((H, 3)))
    assert (s[..., k1] == s[..., k2]).all()
    assert (k_star == k1).all()


def test_argmax_decided_on_fp32_scores():
    """Two scores that differ in fp64 by less than half an fp32 ulp round to
    the same fp32 value: the decision, taken in fp32, is a tie and goes to the
    lower index (an fp64 argmax would take the higher one)."""
    H, K, d, L = 1, 3, 2, 1
    u = np.zeros((1, H, L, d))
    u[..., 0] = 1.0
    u[..., 1] = 2.0 ** -30
    W = np.zeros((H, K, d))
    W[0, 0] = [1.0, 0.0]                 # score 1
    W[0, 2] = [1.0, 1.0]                 # score 1 + 2^-30: distinct in fp64, equal in fp32
    k_star, _, s = oracle.select(u, W, np.zeros((H, 1, d)), np.zeros((H, 1)))
    assert s[0, 0, 0, 2] > s[0, 0, 0, 0] and np.float32(s[0, 0, 0, 2]) == np.float32(s[0, 0, 0, 0])
    assert k_star[0, 0, 0] == 0


# --------------------------------------------------------------------------
# F10: logistic identities
# --------------------------------------------------------------------------

def test_sigmoid_identities():
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(math.log(3.0)) - 0.75) <= 2e-16
    assert abs(oracle.sigmoid(-math.log(3.0)) - 0.25) <= 2e-16
    assert abs(oracle.sigmoid(math.log(7.0)) - 0.875) <= 2e-16
    x = np.linspace(-30, 30, 2001)
    s = oracle.sigmoid(x)
    np.testing.assert_allclose(oracle.sigmoid(-x), 1.0 - s, rtol=0, atol=2e-16)
    assert (np.diff(s) >= 0).all()
    ref = np.array([1.0 / (1.0 + math.exp(-v)) for v in x])
    np.testing.assert_allclose(s, ref, rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# F11: selection indexing over batch, head and the shared layout
# --------------------------------------------------------------------------

def test_selection_indexing_per_head():
    """Head h of batch b sees u = 3 e_{(b+h) mod K} + small noise; W_sel = I-ish
    per head with a head-dependent permutation, so the expected k* is known."""
    rng = np.random.default_rng(11)
    B, H, L, K, N, d = 3, 4, 5, 6, 3, 8
    perms = [rng.permutation(K) for _ in range(H)]
    W = np.zeros((H, K, d))
    for h in range(H):
        W[h, perms[h], np.arange(K)] = 1.0       # score k reads channel perms^-1...
    u = rng.standard_normal((B, H, L, d)) * 0.01
    expect = np.zeros((B, H, L), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            ch = (b + h) % K
            u[b, h, :, ch] += 3.0
            expect[b, h] = perms[h][ch]
    b_d = rng.standard_normal((H, N))
    k_star, D, _ = oracle.select(u, W, np.zeros((H, N, d)), b_d)
    assert np.array_equal(k_star, expect)
    np.testing.assert_allclose(D, np.broadcast_to(1 / (1 + np.exp(-b_d))[None, :, None, :], D.shape),
                               rtol=1e-15)


def test_selection_indexing_shared():
    rng = np.random.default_rng(12)
    B, H, L, K, N, d = 2, 5, 7, 4, 3, 8
    u = rng.standard_normal((B, L, d)) * 0.01
    sym = rng.integers(0, K, size=(B, L))
    u[np.arange(B)[:, None], np.arange(L)[None], sym] += 3.0
    W = np.zeros((H, K, d))
    for h in range(H):
        for k in range(K):
            W[h, k, (k + h) % K] = 1.0                # head h: score k reads channel k+h
    k_star, _, _ = oracle.select(u, W, np.zeros((H, N, d)), np.zeros((H, N)), u_shared=True)
    for h in range(H):
        assert np.array_equal(k_star[:, h], (sym - h) % K)


def test_scores_bruteforce():
    rng = np.random.default_rng(13)
    B, H, L, K, d = 2, 3, 4, 5, 6
    u = rng.standard_normal((B, H, L, d))
    W = rng.standard_normal((H, K, d))
    s = oracle.scores(u, W, False)
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for k in range(K):
                    ref = math.fsum(W[h, k, c] * u[b, h, t, c] for c in range(d))
                    assert abs(s[b, h, t, k] - ref) <= 1e-14
    us = rng.standard_normal((B, L, d))
    s2 = oracle.scores(us, W, True)
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for k in range(K):
                    ref = math.fsum(W[h, k, c] * us[b, t, c] for c in range(d))
                    assert abs(s2[b, h, t, k] - ref) <= 1e-14


# --------------------------------------------------------------------------
# planted mistakes: each plausible slip must trip at least one pin
# --------------------------------------------------------------------------

def _transposed_scan(k_star, dict_idx, D, Bu, C, h0=None):
    """Row-one-hot reading (gather instead of scatter)."""
    B, H, L = k_star.shape
    x = np.array(h0, dtype=float)
    y = np.zeros((B, H, L))
    for t in range(L):
        for b in range(B):
            for h in range(H):
                idx = dict_idx[h, k_star[b, h, t]]
                x[b, h] = D[b, h, t] * x[b, h][idx] + Bu[b, h, t]
                y[b, h, t] = (C[h] * x[b, h]).sum()
    return y, x


def _y_before_update(k_star, dict_idx, D, Bu, C, h0=None):
    B, H, L = k_star.shape
    x = np.array(h0, dtype=float)
    y = np.zeros((B, H, L))
    for t in range(L):
        y[:, :, t] = (C[None] * x).sum(-1)
        for b in range(B):
            for h in range(H):
                A = oracle.transition_matrix(dict_idx[h, k_star[b, h, t]], D[b, h, t])
                x[b, h] = A @ x[b, h] + Bu[b, h, t]
    return y, x


def _scale_after_move(k_star, dict_idx, D, Bu, C, h0=None):
    """A = D P (diagonal applied after the move) instead of P D."""
    B, H, L = k_star.shape
    x = np.array(h0, dtype=float)
    y = np.zeros((B, H, L))
    for t in range(L):
        for b in range(B):
            for h in range(H):
                P = oracle.transition_matrix(dict_idx[h, k_star[b, h, t]], np.ones(D.shape[-1]))
                x[b, h] = D[b, h, t] * (P @ x[b, h]) + Bu[b, h, t]
                y[b, h, t] = (C[h] * x[b, h]).sum()
    return y, x


@pytest.mark.parametrize("wrong", [_transposed_scan, _y_before_update, _scale_after_move])
def test_pins_catch_planted_scan_mistakes(wrong):
    g, _, args = _hand_scan()
    y, hL = wrong(*args)
    assert y[0, 0].tolist() != g["expected_y"] or hL[0, 0].tolist() != g["expected_h_L"]


def test_pins_catch_sign_and_tie_mistakes():
    wrong_sigmoid = lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, float)))   # noqa: E731
    assert abs(wrong_sigmoid(math.log(3.0)) - 0.75) > 0.1
    s = np.array([1.0, 3.0, 3.0, 2.0])
    assert int(np.argmax(s)) == 1
    assert int(len(s) - 1 - np.argmax(s[::-1])) != 1      # "last maximum" would fail F9

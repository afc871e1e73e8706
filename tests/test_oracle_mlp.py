"""Pins of the oracle's activation (GELU) and layer-normalisation LAMP, and of
its PS(mu) matrix product, against what the mathematics fixes (no GPU).

Every function of lamp_mlp_oracle.c is checked against something other than
its own formula: an identity of the tanh GELU, the erf GELU within the
approximation's known error, the oracle's own GELU through finite
differences (for the derivative), numpy's layer normalisation, brute-force
minimal selections, a numpy float32 sequential loop (for the product's
layout at mu = 23), and the pinned PS(mu) dot.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build(force=False)


# ---------------------------------------------------------------------------
# GELU (tanh form) and its derivative
# ---------------------------------------------------------------------------
def test_gelu_odd_identity_and_limits():
    # tanh is odd, so GELU(-y) = GELU(y) - y for the tanh form
    for y in np.linspace(-8, 8, 161):
        assert oracle.gelu(-y) == pytest.approx(oracle.gelu(y) - y, rel=1e-13, abs=1e-13)
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(12.0) == pytest.approx(12.0, rel=1e-15)
    assert abs(oracle.gelu(-12.0)) < 1e-30


def test_gelu_close_to_erf_gelu():
    # the tanh form approximates y Phi(y); the published maximum deviation
    # is below 1e-3 in absolute value (a mistyped constant breaks it)
    ys = np.linspace(-6, 6, 2001)
    dev = max(abs(oracle.gelu(y) - 0.5 * y * (1 + math.erf(y / math.sqrt(2)))) for y in ys)
    assert dev < 1e-3
    assert dev > 1e-6   # and it is the tanh form, not the erf form


def test_gelu_grad_matches_finite_differences():
    for y in list(np.linspace(-7, 7, 57)) + [-0.7518, 1e-3, -1e-3]:
        h = 1e-5 * max(1.0, abs(y))
        fd = (oracle.gelu(y + h) - oracle.gelu(y - h)) / (2 * h)
        assert oracle.gelu_grad(y) == pytest.approx(fd, rel=1e-7, abs=1e-9)


def test_gelu_criterion_closed_forms():
    assert oracle.gelu_criterion(0.0) == 0.0
    assert oracle.gelu_criterion(6.0) == pytest.approx(6.0, rel=1e-6)   # GELU' -> 1
    assert oracle.gelu_criterion(-6.0) < 1e-7                          # GELU' -> 0
    # the minimum of GELU (GELU' = 0) near y = -0.7518 has a vanishing criterion
    ys = np.linspace(-0.8, -0.7, 20001, dtype=np.float32)
    c = np.array([oracle.gelu_criterion(y) for y in ys])
    assert c.min() < 1e-4 * c.max()


# ---------------------------------------------------------------------------
# PS(mu) matrix product
# ---------------------------------------------------------------------------
def test_ps_gemm_layout_and_fp32_case():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((5, 37), dtype=np.float32)
    W = rng.standard_normal((7, 37), dtype=np.float32)
    ylo, yref = oracle.ps_gemm(X, W, mu=23)
    # mu = 23 is FP32: both equal a float32 loop in d order (multiply, add)
    ref = np.zeros((5, 7), np.float32)
    for d in range(37):
        ref = (ref + np.outer(X[:, d], W[:, d]).astype(np.float32)).astype(np.float32)
    assert (ylo.view(np.uint32) == ref.view(np.uint32)).all()
    assert (yref.view(np.uint32) == ref.view(np.uint32)).all()
    ylo4, _ = oracle.ps_gemm(X, W, mu=4)
    for i in range(5):
        for j in range(7):
            assert ylo4[i, j] == np.float32(oracle.ps_dot(X[i], W[j], 4))


# ---------------------------------------------------------------------------
# GELU LAMP
# ---------------------------------------------------------------------------
def mlp_case(M=12, N=96, K=256, mu=4, seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    W = (rng.standard_normal((N, K), dtype=np.float32) / np.float32(16.0)).astype(np.float32)
    return oracle.ps_gemm(X, W, mu=mu)


def bits(mask, N):
    return np.unpackbits(mask.view(np.uint8), bitorder="little").reshape(mask.shape[0], -1)[:, :N]


def test_gelu_lamp_limits_and_structure():
    ylo, yref = mlp_case()
    M, N = ylo.shape
    r = oracle.gelu_lamp(ylo, yref, tau=np.inf)
    assert r["count"].sum() == 0
    np.testing.assert_array_equal(r["ymix"], ylo)
    np.testing.assert_allclose(r["err"], r["err_lowp"], rtol=0, atol=0)
    r0 = oracle.gelu_lamp(ylo, yref, tau=0.0)
    sel0 = bits(r0["mask"], N).astype(bool)
    assert (sel0 == (ylo != 0)).all()   # tau = 0: every nonzero score
    prev = None
    for tau in (1e-3, 1e-2, 1e-1, 1.0):
        r = oracle.gelu_lamp(ylo, yref, tau=tau)
        sel = bits(r["mask"], N).astype(bool)
        assert (sel.sum(1) == r["count"]).all()
        np.testing.assert_array_equal(r["ymix"], np.where(sel, yref, ylo))
        assert (sel == (r["crit"] > np.float64(np.float32(tau)))).all()
        assert (r["err"] <= r["err_lowp"] + 1e-15).all()
        if prev is not None:
            assert (sel <= prev).all()   # masks nested in tau
        prev = sel


def test_gelu_lamp_beats_random_selection():
    """The pages' selectivity claim, for the activation rule: at the same
    count, the rule's choice leaves less error than a random one."""
    ylo, yref = mlp_case(M=40, N=128, K=512, seed=5)
    r = oracle.gelu_lamp(ylo, yref, tau=0.3)
    k = r["count"]
    rng = np.random.default_rng(0)
    g = np.vectorize(oracle.gelu)
    e_rand = 0.0
    for i in range(ylo.shape[0]):
        pick = rng.choice(ylo.shape[1], k[i], replace=False)
        mix = ylo[i].copy()
        mix[pick] = yref[i, pick]
        e_rand += np.abs(g(mix.astype(np.float64)) - g(yref[i].astype(np.float64))).sum()
    assert 0 < k.sum() < ylo.size / 2
    assert r["err"].sum() < 0.5 * e_rand


# ---------------------------------------------------------------------------
# LayerNorm LAMP
# ---------------------------------------------------------------------------
def np_layer_norm(y, gamma, beta, eps):
    y = y.astype(np.float64)
    m = y.mean(-1, keepdims=True)
    v = y.var(-1, keepdims=True)
    return gamma * (y - m) / np.sqrt(v + eps) + beta


def test_ln_output_matches_numpy_layer_norm():
    ylo, yref = mlp_case(N=64)
    rng = np.random.default_rng(1)
    g = (1 + 0.1 * rng.standard_normal(64)).astype(np.float32)
    b = (0.1 * rng.standard_normal(64)).astype(np.float32)
    r = oracle.ln_lamp(ylo, yref, g, b, eps=1e-5, tau=np.inf)
    assert r["count"].sum() == 0
    np.testing.assert_allclose(r["out"], np_layer_norm(ylo, g, b, 1e-5), rtol=2e-6, atol=1e-6)
    r0 = oracle.ln_lamp(ylo, yref, g, b, eps=1e-5, tau=0.0)
    assert (r0["count"] == (ylo != 0).sum(1)).all()
    np.testing.assert_allclose(r0["out"], np_layer_norm(yref, g, b, 1e-5), rtol=2e-6, atol=1e-6)
    assert (r0["err"] == 0).all()
    # the error measures are the l2 distances to the all-FP32 output
    e_lo = np.linalg.norm(np_layer_norm(ylo, g, b, 1e-5) - np_layer_norm(yref, g, b, 1e-5), axis=1)
    np.testing.assert_allclose(r["err_lowp"], e_lo, rtol=1e-9)


def test_ln_greedy_is_minimal_by_brute_force():
    """The selection is the smallest set meeting ||y_U||_2 <= tau sigma sqrt(n):
    every smaller set of any composition violates it (exhaustive, n = 10)."""
    rng = np.random.default_rng(7)
    n = 10
    g = np.ones(n, np.float32)
    b = np.zeros(n, np.float32)
    for trial in range(40):
        ylo = (rng.standard_normal((1, n)) * np.exp(rng.uniform(-2, 2, (1, n)))).astype(np.float32)
        yref = ylo + np.float32(1e-3)
        tau = float(rng.uniform(0.05, 0.9))
        r = oracle.ln_lamp(ylo, yref, g, b, eps=1e-5, tau=tau)
        sel = bits(r["mask"], n)[0].astype(bool)
        y = ylo[0].astype(np.float64)
        T2 = np.float64(np.float32(tau)) ** 2 * (y.var() + np.float64(np.float32(1e-5))) * n
        assert (y[~sel] ** 2).sum() <= T2 * (1 + 1e-12)
        k = int(sel.sum())
        assert k == r["count"][0]
        for kk in range(k):
            for S in itertools.combinations(range(n), kk):
                rest = np.ones(n, bool)
                rest[list(S)] = False
                assert (y[rest] ** 2).sum() > T2 * (1 - 1e-12)


def test_ln_ties_go_to_the_lower_index():
    y = np.array([[3.0, -2.0, 2.0, 2.0, -2.0, 0.5, 0.25, 0.0]], np.float32)
    g = np.ones(8, np.float32)
    b = np.zeros(8, np.float32)
    # tau such that exactly three components must be recomputed: 3 and two of the 2s
    v = y[0].astype(np.float64).var() + np.float64(np.float32(1e-5))
    rest_after_3 = 2 * 4.0 + 0.25 + 0.0625
    rest_after_2 = rest_after_3 + 4.0
    T2 = 0.5 * (rest_after_3 + rest_after_2)
    tau = math.sqrt(T2 / (v * 8))
    r = oracle.ln_lamp(y, y, g, b, eps=1e-5, tau=tau)
    sel = bits(r["mask"], 8)[0].astype(bool)
    assert sel.tolist() == [True, True, True, False, False, False, False, False]


def test_ln_lamp_beats_random_selection():
    ylo, yref = mlp_case(M=40, N=128, K=512, seed=9)
    g = np.ones(128, np.float32)
    b = np.zeros(128, np.float32)
    r = oracle.ln_lamp(ylo, yref, g, b, eps=1e-5, tau=0.8)
    k = r["count"]
    rng = np.random.default_rng(0)
    e_rand = 0.0
    for i in range(ylo.shape[0]):
        pick = rng.choice(128, k[i], replace=False)
        mix = ylo[i:i + 1].copy()
        mix[0, pick] = yref[i, pick]
        e_rand += np.linalg.norm(np_layer_norm(mix, g, b, 1e-5) - np_layer_norm(yref[i:i + 1], g, b, 1e-5))
    assert 0 < k.sum() < ylo.size / 2
    # the bound the rule minimises weighs components by magnitude; the PS(mu)
    # error of a long dot is not purely relative, so the margin is modest
    assert r["err"].sum() < e_rand


def test_ln_infinite_tau_on_a_constant_row_selects_nothing():
    """tau = +inf recomputes nothing, also where sigma = 0 (eps = 0, a
    constant row) makes tau^2 sigma^2 n undefined."""
    y = np.full((2, 16), 0.75, np.float32)
    g = np.ones(16, np.float32)
    b = np.zeros(16, np.float32)
    r = oracle.ln_lamp(y, y, g, b, eps=0.0, tau=np.inf)
    assert (r["count"] == 0).all()
    r0 = oracle.ln_lamp(y, y, g, b, eps=0.0, tau=0.0)
    assert (r0["count"] == 16).all()

"""Pins of the oracle's blocked ("packed") PS(mu) accumulation order (no GPU).

The order is a reading (LAMP summary, "Significance": packed low-precision
accumulation in hardware); it is pinned by hand-derived cases of its
definition (tests/golden/ps_blocked_cases.txt), by the two degenerate block
widths that reduce to the pinned sequential dot, by mu = 23 against a numpy
float32 blocked sum, by the first-order error bound of blocked summation
(Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed., section
4.2), and by its plumbing into the attention rows and the matrix product.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ps_blocked_cases.txt")


@pytest.fixture(scope="module", autouse=True)
def built():
    oracle.build(force=False)


def golden_cases():
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        mu, block, exp, qs, ks = line.split()
        q = np.array([float.fromhex(x) if "x" in x else float(x) for x in qs.split(",")], np.float32)
        k = np.array([float.fromhex(x) if "x" in x else float(x) for x in ks.split(",")], np.float32)
        yield int(mu), int(block), float.fromhex(exp), q, k


def test_golden_cases():
    n = 0
    for mu, block, exp, q, k in golden_cases():
        got = oracle.ps_dot_blocked(q, k, mu, block)
        assert got == exp, (mu, block, q, got, exp)
        n += 1
    assert n == 12


@pytest.mark.parametrize("mu", [4, 7, 10, 23])
def test_degenerate_blocks_are_sequential(mu):
    rng = np.random.default_rng(mu)
    for D in (1, 5, 64, 100):
        q = rng.standard_normal(D).astype(np.float32)
        k = rng.standard_normal(D).astype(np.float32)
        seq = oracle.ps_dot(q, k, mu)
        for b in (0, 1, D, D + 7, 4096):
            assert oracle.ps_dot_blocked(q, k, mu, b) == seq


def test_mu23_is_float32_blocked_summation():
    rng = np.random.default_rng(2)
    for D, b in ((64, 4), (64, 16), (100, 8), (37, 32), (200, 64)):
        q = rng.standard_normal(D).astype(np.float32)
        k = rng.standard_normal(D).astype(np.float32)
        acc = np.float32(0.0)
        for d0 in range(0, D, b):
            part = np.float32(0.0)
            for d in range(d0, min(d0 + b, D)):
                part = np.float32(part + np.float32(q[d] * k[d]))
            acc = np.float32(acc + part)
        assert np.float32(oracle.ps_dot_blocked(q, k, 23, b)) == acc


def test_order_matters_and_runs_compose():
    """Different widths give different results on a generic input, and the
    result is the fold of the run sums (each run a sequential PS dot)."""
    rng = np.random.default_rng(3)
    D = 64
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    vals = {b: oracle.ps_dot_blocked(q, k, 4, b) for b in (0, 2, 4, 8, 16, 32)}
    assert len(set(vals.values())) >= 3
    for b in (2, 4, 8, 16, 32):
        acc = 0.0
        for d0 in range(0, D, b):
            acc = oracle.rn_mu(acc + oracle.ps_dot(q[d0:d0 + b], k[d0:d0 + b], 4), 4)
        assert acc == vals[b]


@pytest.mark.parametrize("mu", [4, 7, 10])
def test_error_bound_of_blocked_summation(mu):
    """|blocked - exact| <= gamma_m sum |q_d k_d| with m = (b - 1) + ceil(D/b)
    + 1 roundings on any path (b - 1 in a run, ceil(D/b) into the
    accumulator, 1 for the product), gamma_m = m u / (1 - m u), u = 2^-(mu+1).
    A run that is dropped or added twice breaks it."""
    rng = np.random.default_rng(10 + mu)
    u = 2.0 ** -(mu + 1)
    checked = 0
    for trial in range(400):
        D = int(rng.integers(2, 60 if mu == 4 else 300))
        b = int(2 ** rng.integers(1, 7))
        m = (b - 1) + math.ceil(D / b) + 1
        if m * u >= 0.5:   # the bound says nothing there
            continue
        checked += 1
        q = rng.standard_normal(D).astype(np.float32)
        k = rng.standard_normal(D).astype(np.float32)
        exact = float(np.dot(q.astype(np.float64), k.astype(np.float64)))
        gamma = m * u / (1 - m * u)
        bound = gamma * float(np.abs(q.astype(np.float64) * k.astype(np.float64)).sum())
        got = oracle.ps_dot_blocked(q, k, mu, b)
        assert abs(got - exact) <= bound * (1 + 1e-12), (D, b)
    assert checked >= 50


def test_blocked_is_more_accurate_on_long_dots():
    """Blocked summation's error grows like b + D/b instead of D: over many
    long dots at mu = 4 its mean error is clearly below the sequential one."""
    rng = np.random.default_rng(4)
    e_seq, e_blk = [], []
    for _ in range(200):
        q = rng.standard_normal(1024).astype(np.float32)
        k = rng.standard_normal(1024).astype(np.float32)
        exact = float(np.dot(q.astype(np.float64), k.astype(np.float64)))
        e_seq.append(abs(oracle.ps_dot(q, k, 4) - exact))
        e_blk.append(abs(oracle.ps_dot_blocked(q, k, 4, 32) - exact))
    assert np.mean(e_blk) < 0.5 * np.mean(e_seq)


def test_plumbing_into_rows_and_products():
    rng = np.random.default_rng(5)
    S, D = 40, 64
    Qh = rng.standard_normal((S, D)).astype(np.float32)
    Kh = rng.standard_normal((S, D)).astype(np.float32)
    Vh = rng.standard_normal((S, D)).astype(np.float32)
    s = oracle.scale(D)
    r0 = oracle.lamp_rows(Qh, Kh, Vh, causal=True, mu=4, tau=0.1, mode=oracle.STRICT)
    r8 = oracle.lamp_rows(Qh, Kh, Vh, causal=True, mu=4, tau=0.1, mode=oracle.STRICT,
                          ps_block=8)
    np.testing.assert_array_equal(r0["yref"], r8["yref"])   # the reference stays sequential
    for i in (0, 7, 39):
        for j in range(i + 1):
            want = np.float32(np.float32(oracle.ps_dot_blocked(Qh[i], Kh[j], 4, 8)) * s)
            assert r8["ylo"][i, j] == want
    assert (r0["ylo"] != r8["ylo"]).any()
    X = rng.standard_normal((5, 96)).astype(np.float32)
    W = rng.standard_normal((6, 96)).astype(np.float32)
    ylo, yref = oracle.ps_gemm(X, W, mu=4, ps_block=16)
    _, yref0 = oracle.ps_gemm(X, W, mu=4)
    np.testing.assert_array_equal(yref, yref0)
    for i in range(5):
        for j in range(6):
            assert ylo[i, j] == np.float32(oracle.ps_dot_blocked(X[i], W[j], 4, 16))

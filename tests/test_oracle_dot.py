"""Pins of the oracle's dot products and score scale.

Source: LAMP technical summary (2601.21623), "Implementation strategy" step 1
(baseline evaluation at low precision) with the PS(mu) format of
"Experimental results"; the uniform FP32 reference of the same section.
Readings: operands stay FP32, every product and every sum is rounded to
PS(mu), d ascending from +0; scores are scaled once, in FP32, by the FP32
value nearest to 1/sqrt(D).
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.test_oracle_rounding import rn_exact


def seq32_numpy(q, k):
    acc = np.float32(0.0)
    for a, b in zip(q, k):
        p = np.float32(a) * np.float32(b)
        acc = np.float32(acc + p)
    return acc


def ps_dot_exact(q, k, mu):
    """Exact PS(mu) dot; once an infinity appears, IEEE float arithmetic
    carries it (inf + -inf = nan), as in the format's overflow reading."""
    acc = Fraction(0)
    for a, b in zip(q, k):
        t = rn_exact(Fraction(float(a)) * Fraction(float(b)), mu)
        if isinstance(acc, float) or isinstance(t, float):
            acc = float(acc) + float(t)
        else:
            acc = rn_exact(acc + t, mu)
    return acc


def _rand_vec(rng, D, emin, emax):
    e = rng.integers(emin, emax + 1, D)
    v = rng.uniform(1.0, 2.0, D) * np.exp2(e) * rng.choice([-1.0, 1.0], D)
    return v.astype(np.float32)


def test_mu23_is_sequential_fp32(orc):
    """PS(23) has FP32's precision and range: the PS dot must equal the plain
    sequential float loop, bit for bit (including subnormal results)."""
    rng = np.random.default_rng(0)
    for trial in range(300):
        D = int(rng.integers(1, 80))
        if trial % 3 == 0:
            q, k = _rand_vec(rng, D, -80, -60), _rand_vec(rng, D, -70, -60)   # subnormal products
        else:
            q, k = rng.standard_normal(D, dtype=np.float32), rng.standard_normal(D, dtype=np.float32)
        want = seq32_numpy(q, k)
        assert np.float32(orc.ps_dot(q, k, 23)).view(np.uint32) == want.view(np.uint32)
        assert orc.seq32_dot(q, k).view(np.uint32) == want.view(np.uint32)


def test_single_term_is_one_rounding(orc):
    rng = np.random.default_rng(1)
    for mu in (1, 4, 7, 10, 16, 22):
        for _ in range(200):
            q, k = _rand_vec(rng, 1, -70, 70), _rand_vec(rng, 1, -70, 70)
            want = rn_exact(Fraction(float(q[0])) * Fraction(float(k[0])), mu)
            assert orc.ps_dot(q, k, mu) == float(want)


@pytest.mark.parametrize("mu", [1, 2, 4, 7, 10, 16, 22, 23])
def test_short_dots_against_exact_rationals(orc, mu):
    rng = np.random.default_rng(100 + mu)
    for trial in range(400):
        D = int(rng.integers(2, 5))
        lo, hi = ((-3, 3), (-30, 30), (-75, -55), (55, 66))[trial % 4]
        q, k = _rand_vec(rng, D, lo, hi), _rand_vec(rng, D, lo, hi)
        want = ps_dot_exact(q, k, mu)
        got = orc.ps_dot(q, k, mu)
        assert got == float(want) or (np.isnan(got) and np.isnan(want)), (mu, q, k, got, want)


def test_order_matters():
    """Sequential rounding, not one rounding of the exact sum: at mu=4,
    1 + 2^-5 + 2^-5 accumulates to 1 (each add ties to even), while the
    reversed order gives 1 + 2^-4."""
    import oracle
    q = np.array([1.0, 2.0 ** -5, 2.0 ** -5], np.float32)
    k = np.ones(3, np.float32)
    assert oracle.ps_dot(q, k, 4) == 1.0
    assert oracle.ps_dot(q[::-1].copy(), k, 4) == 1.0 + 2.0 ** -4


def test_accumulator_starts_at_plus_zero(orc):
    q = np.array([-0.0, -0.0], np.float32)
    k = np.array([1.0, 1.0], np.float32)
    r = orc.ps_dot(q, k, 4)
    assert r == 0.0 and np.copysign(1.0, r) == 1.0


def test_scale_is_nearest_fp32_to_inverse_sqrt(orc):
    for D in range(1, 257):
        s = orc.scale(D)
        sf = Fraction(float(s))
        ulp = Fraction(float(np.spacing(s)))
        lo, hi = sf - ulp / 2, sf + ulp / 2
        assert lo * lo <= Fraction(1, D) <= hi * hi, D
    assert orc.scale(64).view(np.uint32) == 0x3E000000
    assert orc.scale(128).view(np.uint32) == 0x3DB504F3

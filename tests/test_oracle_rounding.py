"""Pins of the oracle's PS(mu) rounding primitive.

The oracle's RN_mu (frexp / nearbyint on doubles) is checked against:
  * hand-derived cases of the format's definition (tests/golden/rn_mu_cases.txt);
  * an independent integer formulation on FP32 bit patterns, exhaustively over
    all 2^32 patterns at mu=4 and over structured sweeps at other mu;
  * exact rational rounding (fractions.Fraction) on random doubles, including
    values far outside the FP32 range.
Format source: LAMP technical summary (2601.21623), "Experimental results"
(PS(mu), mu mantissa bits); reading: FP32 exponent range, ties to even.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rn_mu_cases.txt")


def rn_exact(x: Fraction, mu: int):
    """Exact rational RN_mu with FP32 range; returns Fraction or +-inf."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    b = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** b > a:
        b -= 1
    while Fraction(2) ** (b + 1) <= a:
        b += 1
    b = max(b, -126)
    qt = Fraction(2) ** (b - mu)
    n = a / qt
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * qt
    if r >= Fraction(2) ** 128:
        return sgn * math.inf
    return sgn * r


def rn_bits_f32(u: np.ndarray, mu: int) -> np.ndarray:
    """Integer RNE on FP32 bit patterns: add half-1 plus the kept LSB, clear."""
    u = u.astype(np.uint64)
    sh = 23 - mu
    if sh == 0:
        return u.astype(np.uint32)
    half = np.uint64(1 << (sh - 1))
    lsb = (u >> np.uint64(sh)) & np.uint64(1)
    r = (u + half - np.uint64(1) + lsb) & np.uint64(~((1 << sh) - 1) & 0xFFFFFFFF)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    return np.where(nan, u, r).astype(np.uint32)


def _parse(tok):
    if tok in ("inf", "-inf"):
        return float(tok)
    return float.fromhex(tok)


def test_golden_cases(orc):
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        mu, x, want = line.split()
        x, want = _parse(x), _parse(want)
        got = orc.rn_mu(np.array([x]), int(mu))[0]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (mu, x.hex(), got, want)
        # the exact rational rounding agrees with the hand derivation too
        ex = rn_exact(Fraction(x), int(mu))
        assert float(ex) == want or (math.isinf(ex) and ex == want)
        n += 1
    assert n >= 30


def _sweep(orc, start: int, count: int, mu: int):
    import ctypes
    from tests.helpers import load
    chk = load("rn_bits_check")
    chk.rn_check_range.restype = ctypes.c_int64
    chk.rn_check_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    fn = ctypes.cast(orc._load().orc_rn_mu, ctypes.c_void_p)
    first = ctypes.c_uint32(0)
    bad = chk.rn_check_range(start, count, mu, fn, ctypes.byref(first))
    assert bad == 0, (mu, bad, hex(first.value))


def _check_bits(orc, bits: np.ndarray, mu: int):
    f = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        got = orc.rn_mu(f.astype(np.float64), mu).astype(np.float32).view(np.uint32)
    want = rn_bits_f32(bits, mu)
    nan = np.isnan(f)
    bad = (got != want) & ~nan
    assert not bad.any(), (mu, hex(int(bits[bad][0])), hex(int(got[bad][0])), hex(int(want[bad][0])))
    assert np.isnan(got.view(np.float32)[nan]).all()


@pytest.mark.slow
def test_exhaustive_fp32_mu4(orc):
    """All 2^32 FP32 bit patterns at mu=4 (the headline precision)."""
    _sweep(orc, 0, 1 << 32, 4)


@pytest.mark.parametrize("mu", [1, 7, 10, 11, 16, 22, 23])
def test_structured_fp32_sweep(orc, mu):
    """Every mantissa in a set of binades that covers subnormals, the smallest
    normal binades, ordinary values and the top of the range, both signs."""
    for e in (0, 1, 2, 60, 126, 127, 128, 129, 200, 253, 254, 255):
        for sign in (0, 0x80000000):
            _sweep(orc, sign | (e << 23), 1 << 23, mu)
    # and the numpy formulation on one binade, as a cross-check of the C one
    _check_bits(orc, np.arange(1 << 23, dtype=np.uint32) | np.uint32(127 << 23), mu)


def test_random_doubles_against_fractions(orc):
    """Doubles that are not FP32 values, including far outside FP32 range."""
    rng = np.random.default_rng(1)
    xs = []
    for lo, hi in ((-160, -120), (-20, 20), (120, 135), (-400, 400)):
        e = rng.integers(lo, hi, 400)
        xs.append(np.ldexp(rng.uniform(1.0, 2.0, 400), e) * rng.choice([-1.0, 1.0], 400))
    xs = np.concatenate(xs)
    for mu in (1, 4, 7, 10, 16, 23):
        got = orc.rn_mu(xs, mu)
        for x, g in zip(xs, got):
            want = rn_exact(Fraction(float(x)), mu)
            assert g == float(want), (mu, float(x).hex(), g, want)

"""CPU checks of the arithmetic premise of the GPU's PS(mu) fast path.

The HIP kernels compute PS(mu) products with one FP32 multiply (for the
exponent), a magic constant and one fused multiply-add, and PS(mu) sums with
an FP32 add followed by round-to-nearest-even to mu fraction bits through
Veltkamp's splitting (three FP32 operations).  A scalar
C emulation of exactly that sequence (tests/helpers/fast_ps_emul.c) is
compared here with the oracle, so a flaw in the premise shows up on the CPU.
These are host-logic tests; the GPU parity tests compare the kernels
themselves with the oracle.
"""
import ctypes
import math

import numpy as np
import pytest

from tests.helpers import load


@pytest.fixture(scope="module")
def emu(orc):
    lib = load("fast_ps_emul")
    lib.emu_ps_score.restype = ctypes.c_float
    lib.emu_ps_score.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_float]
    lib.check_products.restype = ctypes.c_int64
    lib.check_products.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
    lib.check_sums_exhaustive.restype = ctypes.c_int64
    lib.check_sums_exhaustive.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.check_split_exhaustive.restype = ctypes.c_int64
    lib.check_split_exhaustive.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
    lib.check_sums_random.restype = ctypes.c_int64
    lib.check_sums_random.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    return lib


def _rn(orc):
    return ctypes.cast(orc._load().orc_rn_mu, ctypes.c_void_p)


@pytest.mark.parametrize("mu", [1, 2, 4, 7, 10])
def test_magic_product_rounding(emu, orc, mu):
    traps = ctypes.c_int64(0)
    bad = emu.check_products(7 + mu, 4_000_000, mu, -40, 40, _rn(orc), ctypes.byref(traps))
    assert bad == 0
    # narrow exponents make products near 1: midpoint traps show up often there
    bad = emu.check_products(11 + mu, 4_000_000, mu, -1, 1, _rn(orc), ctypes.byref(traps))
    assert bad == 0
    assert traps.value > 0 or mu <= 2   # the double-rounding trap was exercised


@pytest.mark.parametrize("mu", [1, 4, 10])
def test_split_rounding_equals_integer_rne_exhaustive(emu, mu):
    """Veltkamp's splitting rounds to nearest, ties to even, on every FP32
    input the fast path can produce (normal magnitudes below 2^100, and +0):
    bit for bit the integer RNE (itself swept against the oracle's RN_mu)."""
    first = ctypes.c_uint32(0)
    bad = emu.check_split_exhaustive(mu, ctypes.byref(first))
    assert bad == 0, (bad, hex(first.value))


@pytest.mark.parametrize("mu,emin,emax", [(1, -20, 20), (4, -20, 20), (7, -12, 12)])
def test_fp32_sum_then_round_exhaustive(emu, orc, mu, emin, emax):
    assert emu.check_sums_exhaustive(mu, emin, emax, _rn(orc)) == 0


@pytest.mark.parametrize("mu", [4, 7, 10])
def test_fp32_sum_then_round_random_wide(emu, orc, mu):
    assert emu.check_sums_random(3 + mu, 2_000_000, mu, -40, 40, _rn(orc)) == 0
    assert emu.check_sums_random(4 + mu, 4_000_000, mu, -15, 15, _rn(orc)) == 0
    assert emu.check_sums_random(5 + mu, 2_000_000, mu, -2, 2, _rn(orc)) == 0


def test_fp32_sum_then_round_fails_beyond_mu10(emu, orc):
    """Above mu=10 the FP32 intermediate is too narrow (24 < 2(mu+1)+1):
    the premise must fail somewhere, which is why mu > 10 takes the exact path."""
    for mu in (11, 12):
        assert emu.check_sums_random(1, 4_000_000, mu, -15, 15, _rn(orc)) > 0


@pytest.mark.parametrize("mu,D,outl", [(4, 64, 8.0), (7, 64, 8.0), (10, 64, 8.0), (4, 128, 16.0),
                                       (1, 64, 1.0), (4, 8, 1.0)])
def test_emulated_scores_match_oracle(emu, orc, mu, D, outl):
    rng = np.random.default_rng(mu * 1000 + D)
    q = rng.standard_normal((3000, D), dtype=np.float32)
    k = rng.standard_normal((3000, D), dtype=np.float32)
    q[:, :2] *= np.float32(outl)
    k[:, :2] *= np.float32(outl)
    s = orc.scale(D)
    for i in range(q.shape[0]):
        qi, ki = np.ascontiguousarray(q[i]), np.ascontiguousarray(k[i])
        got = np.float32(emu.emu_ps_score(qi.ctypes.data, ki.ctypes.data, D, mu, s))
        want = np.float32(np.float32(orc.ps_dot(qi, ki, mu)) * s)
        assert got.view(np.uint32) == want.view(np.uint32), (i, got, want)


@pytest.fixture(scope="module")
def exp_emu():
    lib = load("exp64_emul")
    lib.emu_exp64_short.restype = ctypes.c_double
    lib.emu_exp64_short.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.max_rel_error.restype = ctypes.c_double
    lib.max_rel_error.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                  ctypes.c_double]
    return lib


@pytest.mark.parametrize("deg,bound", [(4, 6.5e-14), (3, 3.7e-11)])
def test_short_exp64_error_bounds(exp_emu, deg, bound):
    """The kernels' shortened double exponentials (Taylor degree 4 for values
    that decide a criterion, 3 for normalising sums and KLs) stay within the
    bounds the truncation and the one-double ln 2 / 64 give, over the whole
    argument range and near 0, where softmax terms concentrate."""
    worst = 0.0
    for seed, lo, hi in [(1, -745.0, 0.0), (2, -20.0, 0.0), (3, -0.05, 0.05), (4, 0.0, 709.0)]:
        worst = max(worst, exp_emu.max_rel_error(deg, seed, 400_000, lo, hi))
    assert worst <= bound, worst
    # the truncation is visible: the degree-3 form is not accidentally exact
    assert deg == 4 or worst > 1e-13


@pytest.mark.parametrize("deg", [3, 4])
def test_short_exp64_special_values(exp_emu, deg):
    assert exp_emu.emu_exp64_short(0.0, deg) == 1.0   # a key at its row maximum
    assert exp_emu.emu_exp64_short(float("-inf"), deg) == 0.0
    assert exp_emu.emu_exp64_short(-800.0, deg) == 0.0
    assert math.isinf(exp_emu.emu_exp64_short(800.0, deg))
    assert math.isnan(exp_emu.emu_exp64_short(float("nan"), deg))

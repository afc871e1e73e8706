"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Bars (the LAMP build's stated tolerances):
  * PS(mu) scores, FP32 scores, y^mix, masks and counts: bit-exact.  A mask
    bit may differ only where the oracle's criterion value sits within a
    relative 1e-12 of tau (an unresolvable tie between two double-precision
    evaluations of exp and a row sum); such ties are counted and reported.
  * probs:  |d| <= 1e-6 |p| + 1e-7
  * out:    |d| <= 1e-6 sum_j p_j |v_jd| + 1e-7   (out can cancel towards 0)
  * KL:     |d| <= 1e-6 |KL| + 1e-7
"""
from __future__ import annotations

import numpy as np

TIE_REL = 1e-12


def valid_mask(S: int, causal: bool, rows=None) -> np.ndarray:
    rows = np.arange(S) if rows is None else np.arange(*rows)
    j = np.arange(S)
    return (j[None, :] <= rows[:, None]) if causal else np.ones((rows.size, S), bool)


def bits_equal(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elementwise bit equality of float32 arrays; NaN matches NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def assert_bits(got, want, valid, what):
    eq = bits_equal(got, want) | ~valid
    if not eq.all():
        idx = np.argwhere(~eq)[:5]
        det = [(tuple(i), float(np.asarray(got)[tuple(i)]), float(np.asarray(want)[tuple(i)]))
               for i in idx]
        raise AssertionError(f"{what}: {(~eq).sum()} of {valid.sum()} differ, e.g. {det}")


def unpack_mask(mask: np.ndarray, S: int) -> np.ndarray:
    m = np.ascontiguousarray(mask).astype(np.uint32)
    bits = np.unpackbits(m.view(np.uint8), bitorder="little")
    return bits.reshape(m.shape[:-1] + (-1,))[..., :S].astype(bool)


def assert_mask(got_words, want_words, crit, tau, S, what="mask"):
    """Mask words equal, except bits at unresolvable ties; padding bits 0."""
    g = unpack_mask(got_words, S)
    w = unpack_mask(want_words, S)
    tie = np.zeros_like(g)
    if np.isfinite(tau) and tau > 0:
        tie = np.abs(crit - tau) <= TIE_REL * tau
    bad = (g != w) & ~tie
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} bits differ, e.g. at {idx.tolist()} "
                             f"crit={[float(crit[tuple(i)]) for i in idx]} tau={tau}")
    # padding bits beyond S must be zero
    W = got_words.shape[-1]
    if W * 32 > S:
        allbits = np.unpackbits(np.ascontiguousarray(got_words).astype(np.uint32).view(np.uint8),
                                bitorder="little").reshape(got_words.shape[:-1] + (-1,))
        assert not allbits[..., S:].any(), f"{what}: padding bits set"
    return int(tie.sum())


def assert_tol(got, want, scale, what, rel=1e-6, abs_=1e-7):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    lim = rel * np.asarray(scale, np.float64) + abs_
    bad = ~(err <= lim)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance, e.g. "
            f"{[(tuple(i), float(got[tuple(i)]), float(want[tuple(i)])) for i in idx]}; "
            f"max err/lim {float((err / lim).max()):.3g}")
    return float((err / lim).max()) if err.size else 0.0


def out_scale(probs64: np.ndarray, V: np.ndarray) -> np.ndarray:
    """sum_j p_j |v_jd| per (row, d), the natural scale of out."""
    return probs64 @ np.abs(V.astype(np.float64))


def assert_out_with_nonfinite(got, want, scale, what="out"):
    """out where V holds infinities or NaN: every non-finite oracle value is
    matched exactly (NaN by NaN, an infinity by the same infinity), every
    finite one within the out tolerance."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    nf = ~np.isfinite(want)
    same = (np.isnan(got) & np.isnan(want)) | (got == want)
    bad = nf & ~same
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} non-finite values differ, e.g. "
                             f"{[(tuple(i), got[tuple(i)], want[tuple(i)]) for i in idx]}")
    assert nf.any() and (~nf).any(), "the case should hold finite and non-finite outputs"
    return assert_tol(got[~nf], want[~nf], np.asarray(scale, np.float64)[~nf], what)

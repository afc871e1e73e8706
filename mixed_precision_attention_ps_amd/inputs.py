"""Seeded synthetic inputs for LAMP attention.

This module only draws random numbers; it holds none of the method's
arithmetic.  It is the one module that serves both the HIP path and the CPU
oracle (tests and the benchmark feed both from it).

Recipe (stands in for GPT-2 activations on OpenWebText, which the LAMP
summary's "Experimental results" section uses and which are not available):
``numpy.random.default_rng(seed)``; Q, K, V drawn in that order as float32
standard normals of shape [B, H, S, D]; Q and K optionally multiplied by a
power-of-two ``qk_std`` (exact); then ``n_outlier`` channel indices drawn with
``rng.choice(D, n_outlier, replace=False)`` and sorted; the same channels of
Q and K (all batches and heads) are multiplied by ``outlier_factor``.  Scaled
outlier channels in both Q and K make the softmax rows peaked.

Matrix-product inputs (``make_mlp``): X [M, K] float32 standard normals (the
normalised activations entering a projection), then W [N, K] standard normals
times ``w_std`` rounded to float32 (GPT-2's initialisation uses 0.02), then
gamma = 1 + 0.1 N(0, 1) and beta = 0.1 N(0, 1) of length N.
"""
from __future__ import annotations

import numpy as np


def make_qkv(B: int, H: int, S: int, D: int, *, n_outlier: int = 0,
             outlier_factor: float = 8.0, qk_std: float = 1.0, seed: int = 0):
    """Return (Q, K, V, outlier_channels) as contiguous float32 arrays."""
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    Q = rng.standard_normal(shape, dtype=np.float32)
    K = rng.standard_normal(shape, dtype=np.float32)
    V = rng.standard_normal(shape, dtype=np.float32)
    if qk_std != 1.0:
        Q *= np.float32(qk_std)
        K *= np.float32(qk_std)
    idx = np.sort(rng.choice(D, n_outlier, replace=False)) if n_outlier > 0 else np.zeros(0, np.int64)
    if n_outlier > 0:
        Q[..., idx] *= np.float32(outlier_factor)
        K[..., idx] *= np.float32(outlier_factor)
    return Q, K, V, idx


def make_mlp(M: int, N: int, K: int, *, w_std: float = 0.02, seed: int = 0):
    """Return (X, W, gamma, beta) as contiguous float32 arrays."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(N)).astype(np.float32)
    return X, W, gamma, beta


def make_special_matrix(rows: int, K: int, *, kind: str, seed: int = 0):
    """One [rows, K] operand outside the normal range, as ``make_special``'s Q."""
    Q, _, _ = make_special(1, 1, rows, K, kind=kind, seed=seed)
    return np.ascontiguousarray(Q[0, 0])


def make_special(B: int, H: int, S: int, D: int, *, kind: str, seed: int = 0):
    """Inputs that leave the normal range on purpose (edge-case parity).

    kind: "tiny"     -- magnitudes spread over [2^-75, 2^-45] (subnormal products)
          "huge"     -- magnitudes spread over [2^40, 2^66] (products overflow)
          "mixed"    -- normal values with a few zeros, tiny and huge entries
          "nonfinite"-- normal values with a few inf / nan entries
          "nonfinite_v" -- Q, K standard normal; V standard normal with a
                      few +inf, -inf and nan entries (about 0.1 %, 0.1 % and
                      0.05 %)
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    sign = lambda: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    if kind == "tiny":
        e = rng.integers(-75, -45, size=shape)
        mk = lambda: (sign() * rng.uniform(1.0, 2.0, shape) * np.exp2(e)).astype(np.float32)
        Q, K = mk(), mk()
    elif kind == "huge":
        e = rng.integers(40, 66, size=shape)
        mk = lambda: (sign() * rng.uniform(1.0, 2.0, shape) * np.exp2(e)).astype(np.float32)
        Q, K = mk(), mk()
    elif kind in ("mixed", "nonfinite"):
        Q = rng.standard_normal(shape, dtype=np.float32)
        K = rng.standard_normal(shape, dtype=np.float32)
        for X in (Q, K):
            u = rng.random(shape)
            X[u < 0.02] = 0.0
            if kind == "mixed":
                X[(u >= 0.02) & (u < 0.03)] *= np.float32(2.0 ** -70)
                X[(u >= 0.03) & (u < 0.035)] *= np.float32(2.0 ** 50)
            else:
                X[(u >= 0.02) & (u < 0.021)] = np.inf
                X[(u >= 0.021) & (u < 0.022)] = -np.inf
                X[(u >= 0.022) & (u < 0.023)] = np.nan
    elif kind == "nonfinite_v":
        Q = rng.standard_normal(shape, dtype=np.float32)
        K = rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError(kind)
    V = rng.standard_normal(shape, dtype=np.float32)
    if kind == "nonfinite_v":
        u = rng.random(shape)
        V[u < 0.001] = np.inf
        V[(u >= 0.001) & (u < 0.002)] = -np.inf
        V[(u >= 0.002) & (u < 0.0025)] = np.nan
    return np.ascontiguousarray(Q), np.ascontiguousarray(K), V

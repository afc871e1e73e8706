"""CPU oracle for LAMP attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and this
package never imports the product.  The two share no code; only the seeded
input generator module serves both.

The arithmetic lives in ``lamp_oracle.c`` (plain C, double precision, one
attention row at a time).  This module compiles it with gcc and wraps it with
ctypes.  Method source: the LAMP technical summary (gist.science, paper
2601.21623), "Theoretical foundation" item 3 (softmax closed form),
"Implementation strategy" steps 1-3 and "Experimental results" (PS(mu),
KL against uniform FP32, random control, relaxed relative-threshold LAMP).

Parity status of each function is recorded with its pins in ``tests/``:
every function here is pinned; the pages' model-level KL-reduction factors
(GPT-2 XL on OpenWebText) are the one "parity unpinned" item, because no
weights or dataset exist here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lamp_oracle.c")
_SRC_MLP = os.path.join(_HERE, "lamp_mlp_oracle.c")
_LIB = os.path.join(_HERE, "liblamp_oracle.so")

STRICT, RELAXED, RANDOM = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-Wall", "-fPIC", "-shared", "-o", tmp, _SRC, _SRC_MLP, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(os.path.getmtime(_SRC),
                                                                os.path.getmtime(_SRC_MLP)):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    lib.orc_rn_mu.restype = ctypes.c_double
    lib.orc_rn_mu.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.orc_rn_mu_array.restype = None
    lib.orc_rn_mu_array.argtypes = [P, P, ctypes.c_int64, ctypes.c_int]
    lib.orc_scale.restype = ctypes.c_float
    lib.orc_scale.argtypes = [ctypes.c_int]
    lib.orc_ps_dot.restype = ctypes.c_double
    lib.orc_ps_dot.argtypes = [P, P, ctypes.c_int, ctypes.c_int]
    lib.orc_ps_dot_blocked.restype = ctypes.c_double
    lib.orc_ps_dot_blocked.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_seq32_dot.restype = ctypes.c_float
    lib.orc_seq32_dot.argtypes = [P, P, ctypes.c_int]
    lib.orc_splitmix64.restype = ctypes.c_uint64
    lib.orc_splitmix64.argtypes = [ctypes.c_uint64]
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_max_threads.argtypes = []
    lib.orc_lamp_rows.restype = ctypes.c_int
    lib.orc_lamp_rows.argtypes = ([P, P, P] + [ctypes.c_int] * 5 + [ctypes.c_float]
                                  + [ctypes.c_int] * 2 + [ctypes.c_uint64] * 2
                                  + [ctypes.c_int] * 3 + [P] * 9)
    lib.orc_ps_gemm.restype = ctypes.c_int
    lib.orc_ps_gemm.argtypes = [P, P] + [ctypes.c_int] * 6 + [P, P]
    lib.orc_gelu.restype = ctypes.c_double
    lib.orc_gelu.argtypes = [ctypes.c_double]
    lib.orc_gelu_grad.restype = ctypes.c_double
    lib.orc_gelu_grad.argtypes = [ctypes.c_double]
    lib.orc_gelu_criterion.restype = ctypes.c_double
    lib.orc_gelu_criterion.argtypes = [ctypes.c_float]
    lib.orc_gelu_lamp.restype = ctypes.c_int
    lib.orc_gelu_lamp.argtypes = ([P, P, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int]
                                  + [P] * 7)
    lib.orc_ln_lamp.restype = ctypes.c_int
    lib.orc_ln_lamp.argtypes = ([P, P, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_int] + [P] * 7)
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def rn_mu(x, mu: int) -> np.ndarray:
    """RN_mu applied elementwise to float64 values."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib.orc_rn_mu_array(_ptr(x), _ptr(y), x.size, int(mu))
    return y


def scale(D: int) -> np.float32:
    return np.float32(_load().orc_scale(int(D)))


def ps_dot(q, k, mu: int) -> float:
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    assert q.shape == k.shape and q.ndim == 1
    return _load().orc_ps_dot(_ptr(q), _ptr(k), q.size, int(mu))


def ps_dot_blocked(q, k, mu: int, block: int) -> float:
    """PS(mu) dot in the blocked order: runs of `block` products summed from
    +0, each run's sum added to the running accumulator."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    assert q.shape == k.shape and q.ndim == 1
    return _load().orc_ps_dot_blocked(_ptr(q), _ptr(k), q.size, int(mu), int(block))


def seq32_dot(q, k) -> np.float32:
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    assert q.shape == k.shape and q.ndim == 1
    return np.float32(_load().orc_seq32_dot(_ptr(q), _ptr(k), q.size))


def splitmix64(state: int) -> int:
    return int(_load().orc_splitmix64(ctypes.c_uint64(state & 0xFFFFFFFFFFFFFFFF)))


def max_threads() -> int:
    return int(_load().orc_max_threads())


def lamp_rows(qh, kh, vh, *, causal: bool, mu: int, tau: float, mode: int,
              seed: int = 0, head_lin: int = 0, row_begin: int = 0, row_end=None,
              block_k: int = 64, ps_block: int = 0, threads: int = 0,
              want=("ylo", "yref", "crit", "mask", "probs", "out", "kl", "kl_lowp", "count")):
    """Rows [row_begin, row_end) of one head.  qh, kh, vh: float32 [S, D].
    ps_block: PS(mu) accumulation order (0 or 1 sequential, else blocked)."""
    lib = _load()
    qh = np.ascontiguousarray(qh, dtype=np.float32)
    kh = np.ascontiguousarray(kh, dtype=np.float32)
    vh = np.ascontiguousarray(vh, dtype=np.float32)
    S, D = qh.shape
    if row_end is None:
        row_end = S
    n = row_end - row_begin
    W = (S + 31) // 32
    shapes = {"ylo": ((n, S), np.float32), "yref": ((n, S), np.float32),
              "crit": ((n, S), np.float64), "mask": ((n, W), np.uint32),
              "probs": ((n, S), np.float32), "out": ((n, D), np.float32),
              "kl": ((n,), np.float64), "kl_lowp": ((n,), np.float64),
              "count": ((n,), np.int32)}
    res = {name: np.zeros(*shapes[name]) for name in want}
    rc = lib.orc_lamp_rows(_ptr(qh), _ptr(kh), _ptr(vh), S, D, int(bool(causal)), int(mu),
                           int(ps_block), ctypes.c_float(np.float32(tau)), int(mode), int(block_k),
                           ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF),
                           ctypes.c_uint64(head_lin), int(row_begin), int(row_end), int(threads),
                           *[_ptr(res.get(k)) for k in ("ylo", "yref", "crit", "mask", "probs",
                                                         "out", "kl", "kl_lowp", "count")])
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return res


def lamp_heads(Q, K, V, *, causal: bool, mu: int, tau: float, mode: int, heads=None,
               rows=None, seed: int = 0, block_k: int = 64, ps_block: int = 0,
               threads: int = 0, want=None):
    """Selected heads of a [B, H, S, D] problem.

    heads: iterable of linear head indices b*H + h (default: all).
    rows:  optional (row_begin, row_end) applied to every head.
    Returns a dict of arrays stacked over the selected heads.
    """
    B, H, S, D = Q.shape
    heads = list(range(B * H)) if heads is None else list(heads)
    rb, re_ = (0, S) if rows is None else rows
    kw = {} if want is None else {"want": want}
    parts = []
    Qf, Kf, Vf = (x.reshape(B * H, S, D) for x in (Q, K, V))
    for hl in heads:
        parts.append(lamp_rows(Qf[hl], Kf[hl], Vf[hl], causal=causal, mu=mu, tau=tau,
                               mode=mode, seed=seed, head_lin=hl, row_begin=rb, row_end=re_,
                               block_k=block_k, ps_block=ps_block, threads=threads, **kw))
    return {k: np.stack([p[k] for p in parts]) for k in parts[0]}


# ---------------------------------------------------------------------------
# Activation (GELU) and layer-normalisation LAMP after a matrix product
# (lamp_mlp_oracle.c).
# ---------------------------------------------------------------------------
def ps_gemm(X, W, *, mu: int, ps_block: int = 0, threads: int = 0):
    """y = X W^T for X [M, K], W [N, K]: (y_lo PS(mu), y_ref sequential FP32);
    ps_block as for lamp_rows."""
    X = np.ascontiguousarray(X, np.float32)
    W = np.ascontiguousarray(W, np.float32)
    M, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K
    ylo = np.empty((M, N), np.float32)
    yref = np.empty((M, N), np.float32)
    rc = _load().orc_ps_gemm(_ptr(X), _ptr(W), M, N, K, int(mu), int(ps_block), int(threads),
                             _ptr(ylo),
                             _ptr(yref))
    if rc != 0:
        raise ValueError("orc_ps_gemm: bad arguments")
    return ylo, yref


def gelu(y: float) -> float:
    return _load().orc_gelu(float(y))


def gelu_grad(y: float) -> float:
    return _load().orc_gelu_grad(float(y))


def gelu_criterion(y) -> float:
    return _load().orc_gelu_criterion(float(np.float32(y)))


def gelu_lamp(ylo, yref, *, tau: float, threads: int = 0):
    """GELU LAMP over rows: dict of crit, mask, ymix, out, count, err, err_lowp."""
    ylo = np.ascontiguousarray(ylo, np.float32)
    yref = np.ascontiguousarray(yref, np.float32)
    M, N = ylo.shape
    W = (N + 31) // 32
    r = {"crit": np.empty((M, N)), "mask": np.empty((M, W), np.uint32),
         "ymix": np.empty((M, N), np.float32), "out": np.empty((M, N), np.float32),
         "count": np.empty(M, np.int32), "err": np.empty(M), "err_lowp": np.empty(M)}
    rc = _load().orc_gelu_lamp(_ptr(ylo), _ptr(yref), M, N, ctypes.c_float(tau), int(threads),
                               *(_ptr(r[k]) for k in ("crit", "mask", "ymix", "out", "count",
                                                      "err", "err_lowp")))
    if rc != 0:
        raise ValueError("orc_gelu_lamp: bad arguments")
    return r


def ln_lamp(ylo, yref, gamma, beta, *, eps: float, tau: float, threads: int = 0):
    """LayerNorm LAMP over rows: dict of mask, ymix, out, count, err, err_lowp,
    margin."""
    ylo = np.ascontiguousarray(ylo, np.float32)
    yref = np.ascontiguousarray(yref, np.float32)
    gamma = np.ascontiguousarray(gamma, np.float32)
    beta = np.ascontiguousarray(beta, np.float32)
    M, N = ylo.shape
    W = (N + 31) // 32
    r = {"mask": np.empty((M, W), np.uint32), "ymix": np.empty((M, N), np.float32),
         "out": np.empty((M, N), np.float32), "count": np.empty(M, np.int32),
         "err": np.empty(M), "err_lowp": np.empty(M), "margin": np.empty(M)}
    rc = _load().orc_ln_lamp(_ptr(ylo), _ptr(yref), M, N, _ptr(gamma), _ptr(beta),
                             ctypes.c_float(eps), ctypes.c_float(tau), int(threads),
                             *(_ptr(r[k]) for k in ("mask", "ymix", "out", "count", "err",
                                                    "err_lowp", "margin")))
    if rc != 0:
        raise ValueError("orc_ln_lamp: bad arguments")
    return r

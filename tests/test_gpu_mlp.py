"""GPU parity of LAMP after a PS(mu) matrix product: the activation (GELU)
rule and the layer-normalisation rule, against the oracle.

Bars: y^lo, y^ref, y^mix, masks and counts bit-exact (a GELU mask bit may
differ only where the oracle's criterion lies within a relative 1e-12 of tau;
a layer-norm row's selection only where the oracle's k* comparison margin is
below 1e-12); outputs within 1e-6 of their scale + 1e-7; row error measures
within 1e-6 relative + 1e-7.
"""
import sys

import numpy as np
import pytest

from mixed_precision_attention_ps_amd.inputs import make_mlp, make_special_matrix
from tests import parity

pytestmark = pytest.mark.gpu

LN_TIE = 1e-12


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_attention_ps_amd import lamp
    lamp.library()
    return torch.device("cuda:0")


def to_dev(dev, *arrs):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrs]


def run_gelu(dev, X, W, *, mu, tau, want_scores=True):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    M, N = X.shape[0], W.shape[0]
    note(f"gelu M={M} N={N} K={X.shape[1]} mu={mu} tau={tau}")
    x, w = to_dev(dev, X, W)
    mask = torch.full((M, (N + 31) // 32), -1, dtype=torch.int32, device=dev)
    err = torch.zeros(M, dtype=torch.float64, device=dev)
    errl = torch.zeros(M, dtype=torch.float64, device=dev)
    cnt = torch.zeros(M, dtype=torch.int32, device=dev)
    ymix = torch.full((M, N), -3.0, device=dev) if want_scores else None
    yref = torch.full((M, N), -3.0, device=dev) if want_scores else None
    out, st = lamp.lamp_gelu_fwd(x, w, mu=mu, tau=tau, recompute_mask=mask, row_err=err,
                                 row_err_lowp=errl, row_count=cnt, scores_mix=ymix,
                                 scores_ref=yref)
    torch.cuda.synchronize()
    g = {"out": out.cpu().numpy(), "mask": mask.cpu().numpy().view(np.uint32),
         "err": err.cpu().numpy(), "err_lowp": errl.cpu().numpy(), "count": cnt.cpu().numpy(),
         "stats": st}
    if want_scores:
        g["ymix"] = ymix.cpu().numpy()
        g["yref"] = yref.cpu().numpy()
    return g


def check_gelu(g, orc, X, W, *, mu, tau, rows=None):
    rows = np.arange(X.shape[0]) if rows is None else np.asarray(rows)
    N = W.shape[0]
    ylo, yref = orc.ps_gemm(X[rows], W, mu=mu)
    r = orc.gelu_lamp(ylo, yref, tau=tau)
    full = np.ones((rows.size, N), bool)
    if "yref" in g:
        parity.assert_bits(g["yref"][rows], yref, full, "FP32 products")
        sel = parity.unpack_mask(r["mask"], N)
        parity.assert_bits(g["ymix"][rows], np.where(sel, yref, ylo), full, "mixed products")
    ties = parity.assert_mask(g["mask"][rows], r["mask"], r["crit"], tau, N)
    assert (g["count"][rows] == r["count"]).all() or ties > 0, "row counts"
    with np.errstate(invalid="ignore"):
        assert_tol_nf(g["out"][rows], r["out"], np.abs(r["out"]), "GELU output")
        assert_tol_nf(g["err"][rows], r["err"], np.abs(r["err"]), "row l1 error")
        assert_tol_nf(g["err_lowp"][rows], r["err_lowp"], np.abs(r["err_lowp"]),
                      "row l1 error (all PS)")
    if rows.size == X.shape[0]:
        st = g["stats"]
        assert st["n_selected"] == r["count"].sum() or ties > 0
        assert st["n_valid"] == X.shape[0] * N
    return r


def assert_tol_nf(got, want, scale, what):
    """Non-finite expected values must be matched exactly (same infinity, or
    NaN for NaN); the finite ones to the tolerance."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    nf = ~np.isfinite(want)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same[nf].all(), f"{what}: {(~same[nf]).sum()} non-finite values differ"
    fin = ~nf
    parity.assert_tol(got[fin], want[fin], np.asarray(scale, np.float64)[fin], what)


def run_ln(dev, X, W, gamma, beta, *, mu, eps, tau, want_scores=True):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    M, N = X.shape[0], W.shape[0]
    note(f"layernorm M={M} N={N} K={X.shape[1]} mu={mu} eps={eps} tau={tau}")
    x, w, gm, bt = to_dev(dev, X, W, gamma, beta)
    mask = torch.full((M, (N + 31) // 32), -1, dtype=torch.int32, device=dev)
    err = torch.zeros(M, dtype=torch.float64, device=dev)
    errl = torch.zeros(M, dtype=torch.float64, device=dev)
    cnt = torch.zeros(M, dtype=torch.int32, device=dev)
    ymix = torch.full((M, N), -3.0, device=dev) if want_scores else None
    yref = torch.full((M, N), -3.0, device=dev) if want_scores else None
    out, st = lamp.lamp_layernorm_fwd(x, w, gm, bt, mu=mu, eps=eps, tau=tau, recompute_mask=mask,
                                      row_err=err, row_err_lowp=errl, row_count=cnt,
                                      scores_mix=ymix, scores_ref=yref)
    torch.cuda.synchronize()
    g = {"out": out.cpu().numpy(), "mask": mask.cpu().numpy().view(np.uint32),
         "err": err.cpu().numpy(), "err_lowp": errl.cpu().numpy(), "count": cnt.cpu().numpy(),
         "stats": st}
    if want_scores:
        g["ymix"] = ymix.cpu().numpy()
        g["yref"] = yref.cpu().numpy()
    return g


def ln_scale(ymix, gamma, beta, eps):
    """|gamma| |normalised y| + |beta| per element, the natural scale of out."""
    y = ymix.astype(np.float64)
    z = (y - y.mean(1, keepdims=True)) / np.sqrt(y.var(1, keepdims=True) + eps)
    return np.abs(gamma.astype(np.float64)) * np.abs(z) + np.abs(beta.astype(np.float64))


def check_ln(g, orc, X, W, gamma, beta, *, mu, eps, tau, rows=None):
    rows = np.arange(X.shape[0]) if rows is None else np.asarray(rows)
    N = W.shape[0]
    ylo, yref = orc.ps_gemm(X[rows], W, mu=mu)
    r = orc.ln_lamp(ylo, yref, gamma, beta, eps=eps, tau=tau)
    full = np.ones((rows.size, N), bool)
    tie = r["margin"] <= LN_TIE
    ok = ~tie
    if "yref" in g:
        parity.assert_bits(g["yref"][rows], yref, full, "FP32 products")
        parity.assert_bits(g["ymix"][rows][ok], r["ymix"][ok], full[ok], "mixed products")
    gm = g["mask"][rows]
    assert (gm[ok] == r["mask"][ok]).all(), "layer-norm masks"
    assert (g["count"][rows][ok] == r["count"][ok]).all(), "row counts"
    # away from ties the mixed rows are equal, so outputs and errors compare
    with np.errstate(invalid="ignore"):
        parity.assert_tol(g["out"][rows][ok], r["out"][ok],
                          ln_scale(r["ymix"], gamma, beta, eps)[ok], "layer-norm output")
    parity.assert_tol(g["err"][rows][ok], r["err"][ok], np.abs(r["err"][ok]), "row l2 error")
    parity.assert_tol(g["err_lowp"][rows], r["err_lowp"], np.abs(r["err_lowp"]),
                      "row l2 error (all PS)")
    # padding bits of the mask are zero
    if gm.shape[1] * 32 > N:
        allbits = np.unpackbits(gm.view(np.uint8), bitorder="little").reshape(gm.shape[0], -1)
        assert not allbits[:, N:].any()
    if rows.size == X.shape[0] and not tie.any():
        assert g["stats"]["n_selected"] == r["count"].sum()
    return r, int(tie.sum())


# ---------------------------------------------------------------------------
def tile_kind(M, N):
    """Which fast-path tile the library picks for an M x N product (64 x 64
    "wide" or 32 x 32 "narrow"): narrow for fewer than 1024 wide tiles when it
    spreads the work-groups clearly more evenly over the 256 CUs.  Documents
    the coverage of the cases below."""
    import math

    def bal(n):
        return n / (256 * math.ceil(n / 256))
    t64 = -(-M // 64) * -(-N // 64)
    t32 = -(-M // 32) * -(-N // 32)
    return "narrow" if t64 < 1024 and bal(t32) > bal(t64) + 0.05 else "wide"


GEMM_CASES = [
    # M, N, K, mu
    (1, 1, 4, 4),
    (70, 130, 256, 4),
    (130, 300, 100, 4),     # narrow tiles, ragged M, N and K
    (33, 97, 100, 7),       # K not a multiple of the 32-wide chunk
    (64, 64, 1600, 10),
    (65, 66, 68, 12),       # exact double path (mu > 10)
    (40, 50, 96, 23),       # FP32 everywhere
]


@pytest.mark.parametrize("M,N,K,mu", GEMM_CASES)
def test_gemm_scores(dev, orc, M, N, K, mu):
    from mixed_precision_attention_ps_amd import lamp
    X, W, _, _ = make_mlp(M, N, K, w_std=0.05, seed=M + N + K)
    note(f"gemm M={M} N={N} K={K} mu={mu}")
    x, w = to_dev(dev, X, W)
    ylo, yref = lamp.lamp_gemm_scores(x, w, mu=mu)
    ol, orf = orc.ps_gemm(X, W, mu=mu)
    full = np.ones((M, N), bool)
    parity.assert_bits(ylo.cpu().numpy(), ol, full, "PS(mu) products")
    parity.assert_bits(yref.cpu().numpy(), orf, full, "FP32 products")


GELU_CASES = [
    # M, N, K, mu, tau
    (1, 1, 4, 4, 0.1),
    (70, 300, 100, 4, 0.05),    # narrow tiles, ragged
    (200, 450, 1600, 7, 0.02),  # narrow tiles
    (70, 130, 256, 4, 0.1),
    (33, 97, 100, 7, 0.05),
    (64, 64, 64, 4, 0.0),
    (129, 200, 1600, 4, 0.02),
    (20, 70, 96, 10, 0.3),
    (31, 65, 128, 12, 0.1),     # exact double path
    (17, 40, 64, 23, 0.1),      # FP32 everywhere
]


@pytest.mark.parametrize("M,N,K,mu,tau", GELU_CASES)
def test_gelu_small(dev, orc, M, N, K, mu, tau):
    X, W, _, _ = make_mlp(M, N, K, w_std=0.05, seed=3 * M + N)
    g = run_gelu(dev, X, W, mu=mu, tau=tau)
    check_gelu(g, orc, X, W, mu=mu, tau=tau)
    if mu <= 10 and tau > 0:
        assert g["stats"]["n_exact_tiles"] == 0


def test_tile_kinds_covered():
    kinds = {tile_kind(M, N) for (M, N, *_rest) in GEMM_CASES + GELU_CASES + LN_CASES}
    assert kinds == {"wide", "narrow"}
    assert tile_kind(1024, 1600) == "narrow" and tile_kind(1024, 2048) == "wide"


@pytest.mark.parametrize("op,M,N,K", [("gemm", 1024, 2048, 64), ("gelu", 1024, 2048, 96),
                                      ("layernorm", 2048, 1024, 64)])
def test_wide_tiles_at_size(dev, orc, op, M, N, K):
    """Products whose 64 x 64 tiles fill the CUs evenly take the wide tiles;
    sampled rows against the oracle."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    assert tile_kind(M, N) == "wide"
    X, W, gamma, beta = make_mlp(M, N, K, w_std=0.1, seed=M + N)
    rows = [0, 1, 63, 64, 500, M - 1]
    if op == "gemm":
        note(f"gemm M={M} N={N} K={K}")
        x, w = to_dev(dev, X, W)
        ylo, yref = lamp.lamp_gemm_scores(x, w, mu=4)
        ol, orf = orc.ps_gemm(X[rows], W, mu=4)
        full = np.ones((len(rows), N), bool)
        parity.assert_bits(ylo.cpu().numpy()[rows], ol, full, "PS(mu) products")
        parity.assert_bits(yref.cpu().numpy()[rows], orf, full, "FP32 products")
    elif op == "gelu":
        g = run_gelu(dev, X, W, mu=4, tau=0.1)
        check_gelu(g, orc, X, W, mu=4, tau=0.1, rows=rows)
    else:
        g = run_ln(dev, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.3)
        _, ties = check_ln(g, orc, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.3, rows=rows)
        assert ties == 0


def test_gelu_tau_infinite(dev, orc):
    X, W, _, _ = make_mlp(40, 100, 128, w_std=0.05, seed=1)
    g = run_gelu(dev, X, W, mu=4, tau=np.inf)
    check_gelu(g, orc, X, W, mu=4, tau=np.inf)
    assert g["count"].sum() == 0
    np.testing.assert_array_equal(g["err"], g["err_lowp"])


@pytest.mark.parametrize("kind", ["tiny", "huge", "mixed"])
def test_gelu_special_inputs(dev, orc, kind):
    """Operands outside the fast path's range take the exact path."""
    X = make_special_matrix(70, 64, kind=kind, seed=2)
    W = make_special_matrix(90, 64, kind=kind, seed=3)
    g = run_gelu(dev, X, W, mu=4, tau=0.1)
    with np.errstate(all="ignore"):
        check_gelu(g, orc, X, W, mu=4, tau=0.1)
    assert g["stats"]["n_exact_tiles"] > 0


@pytest.mark.parametrize("op", ["gelu", "layernorm"])
def test_mixed_fast_and_exact_blocks(dev, orc, op):
    """One 64-row block of x and one of W hold values outside the fast path's
    range: their tiles go to the exact path, every other tile to the (narrow)
    fast tiles, and the two must agree with the oracle together."""
    M, N, K = 130, 300, 96
    assert tile_kind(M, N) == "narrow"
    X, W, gamma, beta = make_mlp(M, N, K, w_std=0.05, seed=11)
    X[70, 5] = np.float32(2.0 ** 45)
    W[200, 3] = np.float32(2.0 ** -60)
    if op == "gelu":
        g = run_gelu(dev, X, W, mu=4, tau=0.1)
        with np.errstate(all="ignore"):
            check_gelu(g, orc, X, W, mu=4, tau=0.1)
    else:
        g = run_ln(dev, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.3)
        with np.errstate(all="ignore"):
            check_ln(g, orc, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.3)
    # x blocks {1} x all W blocks + W block {3} x the other x blocks
    assert g["stats"]["n_exact_tiles"] == 5 + 2


def test_gelu_workspace_and_stream(dev, orc):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    X, W, _, _ = make_mlp(100, 150, 128, w_std=0.05, seed=4)
    ref = run_gelu(dev, X, W, mu=4, tau=0.05, want_scores=False)
    x, w = to_dev(dev, X, W)
    nbytes = lamp.lamp_mlp_workspace_bytes(100, 150, 128, "gelu")
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, st = lamp.lamp_gelu_fwd(x, w, mu=4, tau=0.05, workspace=ws)
    s.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref["out"])
    assert st["n_selected"] == ref["stats"]["n_selected"]


LN_CASES = [
    # M, N, K, mu, eps, tau
    (1, 1, 4, 4, 1e-5, 0.1),        # one component: var 0, sigma^2 = eps
    (5, 64, 128, 4, 1e-5, 0.1),
    (70, 300, 256, 4, 1e-5, 0.3),
    (33, 97, 100, 7, 1e-5, 0.05),
    (9, 1600, 640, 4, 1e-5, 0.2),
    (3, 8192, 64, 4, 1e-5, 0.2),    # the largest row
    (20, 70, 96, 10, 0.0, 0.5),
    (31, 65, 128, 12, 1e-5, 0.1),   # exact double path
    (17, 40, 64, 23, 1e-5, 0.1),    # FP32 everywhere
]


@pytest.mark.parametrize("M,N,K,mu,eps,tau", LN_CASES)
def test_layernorm_small(dev, orc, M, N, K, mu, eps, tau):
    X, W, gamma, beta = make_mlp(M, N, K, w_std=0.05, seed=5 * M + N)
    g = run_ln(dev, X, W, gamma, beta, mu=mu, eps=eps, tau=tau)
    _, ties = check_ln(g, orc, X, W, gamma, beta, mu=mu, eps=eps, tau=tau)
    assert ties <= 1


@pytest.mark.parametrize("tau", [0.0, np.inf])
def test_layernorm_tau_limits(dev, orc, tau):
    X, W, gamma, beta = make_mlp(30, 200, 128, w_std=0.05, seed=6)
    g = run_ln(dev, X, W, gamma, beta, mu=4, eps=1e-5, tau=tau)
    check_ln(g, orc, X, W, gamma, beta, mu=4, eps=1e-5, tau=tau)
    if tau == np.inf:
        assert g["count"].sum() == 0
        np.testing.assert_allclose(g["err"], g["err_lowp"], rtol=1e-12)
    else:
        # every component with y^lo != 0 (an exact zero of the PS(mu) sum
        # leaves nothing to bound, so it stays)
        assert g["count"].sum() > 0.99 * 30 * 200


def test_layernorm_equal_magnitudes(dev, orc):
    """Equal |y| on either side of the cut go to the lower index: y = x W^T
    with W rows that repeat (and negate) so a row holds many equal
    magnitudes."""
    X, W0, gamma, beta = make_mlp(16, 8, 64, w_std=0.05, seed=8)
    W = np.concatenate([W0, -W0, W0, W0[::-1]], 0)
    gamma, beta = np.ones(32, np.float32), np.zeros(32, np.float32)
    for tau in (0.2, 0.5, 0.9):
        g = run_ln(dev, X, W, gamma, beta, mu=4, eps=1e-5, tau=tau)
        check_ln(g, orc, X, W, gamma, beta, mu=4, eps=1e-5, tau=tau)


@pytest.mark.parametrize("kind", ["tiny", "mixed"])
def test_layernorm_special_inputs(dev, orc, kind):
    X = make_special_matrix(40, 64, kind=kind, seed=4)
    W = make_special_matrix(300, 64, kind=kind, seed=5)
    gamma, beta = np.ones(300, np.float32), np.zeros(300, np.float32)
    g = run_ln(dev, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.1)
    with np.errstate(all="ignore"):
        check_ln(g, orc, X, W, gamma, beta, mu=4, eps=1e-5, tau=0.1)
    assert g["stats"]["n_exact_tiles"] > 0


# ---------------------------------------------------------------------------
# Full-size workloads, one call each, sampled rows against the oracle
# ---------------------------------------------------------------------------
SAMPLE_ROWS = [0, 1, 63, 64, 511, 1000, 1023]


def test_gelu_fullsize(dev, orc):
    from mixed_precision_attention_ps_amd.configs import MLP_WORKLOADS, tau_for
    w = MLP_WORKLOADS["gelu_gpt2_xl_mlp"]
    X, W, _, _ = w.inputs()
    tau = tau_for(w.name, "gelu", 4, 0.016)
    g = run_gelu(dev, X, W, mu=4, tau=tau)
    check_gelu(g, orc, X, W, mu=4, tau=tau, rows=SAMPLE_ROWS)
    rate = g["stats"]["n_selected"] / g["stats"]["n_valid"]
    assert 0.005 < rate < 0.05


def test_layernorm_fullsize(dev, orc):
    from mixed_precision_attention_ps_amd.configs import MLP_WORKLOADS, tau_for
    w = MLP_WORKLOADS["ln_gpt2_xl"]
    X, W, gamma, beta = w.inputs()
    tau = tau_for(w.name, "layernorm", 4, 0.016)
    g = run_ln(dev, X, W, gamma, beta, mu=4, eps=w.eps, tau=tau, want_scores=True)
    _, ties = check_ln(g, orc, X, W, gamma, beta, mu=4, eps=w.eps, tau=tau, rows=SAMPLE_ROWS)
    assert ties == 0
    rate = g["stats"]["n_selected"] / g["stats"]["n_valid"]
    assert 0.005 < rate < 0.05

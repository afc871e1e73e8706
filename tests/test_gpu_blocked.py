"""GPU parity of the blocked ("packed") PS(mu) accumulation order.

lamp_params.ps_block = b sums the products of each run of b consecutive head
dimension (or input) positions from +0 in PS(mu) and adds each run's sum into
the running accumulator (LAMP summary, "Significance"; the order is a reading
the oracle states in orc_ps_dot_blocked).  Every path that forms y^lo takes
it: the attention score tiles (strict, relaxed, random), decode, and the
matrix product before GELU / layer normalisation.  Bars as everywhere: y^lo,
y^mix, y^ref, masks and counts bit-exact; probabilities, outputs and errors
within the stated tolerances.
"""
import numpy as np
import pytest

from mixed_precision_attention_ps_amd.inputs import make_mlp, make_qkv, make_special
from tests import parity
from tests.test_gpu_decode import check as check_decode
from tests.test_gpu_mlp import check_gelu, check_ln, note
from tests.test_gpu_parity import compare_full, run_gpu, run_orc

pytestmark = pytest.mark.gpu

STRICT, RELAXED, RANDOM = 0, 1, 2


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_attention_ps_amd import lamp
    lamp.library()
    return torch.device("cuda:0")


ATTN_CASES = [
    # B, H, S, D, causal, mu, mode, tau, block
    (1, 2, 200, 64, True, 4, STRICT, 0.05, 4),
    (1, 2, 200, 64, True, 4, STRICT, 0.05, 8),
    (1, 1, 130, 64, False, 4, STRICT, 0.05, 16),
    (1, 2, 200, 64, True, 4, STRICT, 0.05, 32),
    (1, 1, 150, 128, True, 4, STRICT, 0.05, 64),     # two runs of 64
    (1, 1, 100, 100, True, 4, STRICT, 0.05, 8),      # a short last run (100 = 12 x 8 + 4)
    (1, 1, 100, 100, True, 4, STRICT, 0.05, 64),     # runs 0..63 | 64..99
    (1, 1, 90, 160, True, 4, STRICT, 0.05, 128),     # runs 0..127 | 128..159
    (1, 2, 200, 64, True, 7, RELAXED, 0.05, 16),
    (1, 1, 150, 128, True, 4, RELAXED, 0.1, 64),
    (1, 1, 130, 96, True, 4, RELAXED, 0.1, 32),      # runs of 32 over three slices
    (1, 2, 200, 64, True, 10, RANDOM, 0.05, 8),
    (1, 1, 100, 64, True, 12, STRICT, 0.05, 16),     # exact double path
    (1, 1, 100, 64, True, 23, STRICT, 0.05, 16),     # mu = 23: blocked FP32 sums
    (1, 1, 100, 64, True, 23, RELAXED, 0.05, 4),
    (1, 1, 1100, 64, True, 4, STRICT, 0.05, 16),     # rows longer than 1024 (multi-kernel path)
]


@pytest.mark.parametrize("B,H,S,D,causal,mu,mode,tau,block", ATTN_CASES)
def test_attention_blocked(dev, orc, B, H, S, D, causal, mu, mode, tau, block):
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=S + D + block)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=mu, tau=tau, mode=mode, seed=3,
                want_probs=S <= 400, ps_block=block)
    heads = None if S <= 400 else [0]
    rows = None if S <= 400 else (S - 40, S)
    r = run_orc(orc, Q, K, V, causal=causal, mu=mu, tau=tau, mode=mode, seed=3, heads=heads,
                rows=rows, ps_block=block)
    compare_full(g, r, Q, V, causal=causal, tau=tau, heads=heads, rows=rows,
                 check_probs=S <= 400)


# the relaxed cases above take the library's choice (two passes for these
# short rows with probabilities); the fused one-pass kernel's blocked variants:
@pytest.mark.parametrize("B,H,S,D,causal,mu,mode,tau,block",
                         [c for c in ATTN_CASES if c[6] == RELAXED])
def test_attention_blocked_relaxed_fused(dev, orc, B, H, S, D, causal, mu, mode, tau, block):
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=S + D + block)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=mu, tau=tau, mode=mode, seed=3,
                ps_block=block, relaxed_path=1)
    r = run_orc(orc, Q, K, V, causal=causal, mu=mu, tau=tau, mode=mode, seed=3, ps_block=block)
    compare_full(g, r, Q, V, causal=causal, tau=tau)


def test_attention_blocked_relaxed_long_rows(dev, orc):
    """Blocked order on rows longer than 1024 keys, relaxed in two passes."""
    S = 1100
    Q, K, V, _ = make_qkv(1, 1, S, 64, n_outlier=2, seed=S + 16)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=0.05, mode=RELAXED, ps_block=16,
                want_probs=False, relaxed_path=2)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=0.05, mode=RELAXED, rows=(S - 40, S),
                ps_block=16)
    compare_full(g, r, Q, V, causal=True, tau=0.05, rows=(S - 40, S), check_probs=False)


def test_blocked_scores_differ_and_reference_does_not(dev, orc):
    """The order changes y^lo (a mask-free check on the raw scores: tau =
    +inf keeps y^mix = y^lo) and leaves the FP32 reference alone; a run as
    long as the head dimension is the sequential order."""
    Q, K, V, _ = make_qkv(1, 1, 128, 64, n_outlier=2, seed=1)
    g0 = run_gpu(dev, Q, K, V, causal=False, mu=4, tau=np.inf, mode=STRICT, want_probs=False)
    g16 = run_gpu(dev, Q, K, V, causal=False, mu=4, tau=np.inf, mode=STRICT, want_probs=False,
                  ps_block=16)
    g64 = run_gpu(dev, Q, K, V, causal=False, mu=4, tau=np.inf, mode=STRICT, want_probs=False,
                  ps_block=64)
    np.testing.assert_array_equal(g0["yref"], g16["yref"])
    assert (g0["ymix"] != g16["ymix"]).mean() > 0.3
    np.testing.assert_array_equal(g0["ymix"], g64["ymix"])
    r = run_orc(orc, Q, K, V, causal=False, mu=4, tau=np.inf, mode=STRICT, ps_block=16)
    valid = np.ones((1, 128, 128), bool)
    parity.assert_bits(g16["ymix"].reshape(1, 128, 128), r["ylo"], valid, "blocked y^lo")


def test_attention_blocked_special_inputs(dev, orc):
    Q, K, V = make_special(1, 2, 150, 64, kind="mixed", seed=7)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=0.1, mode=STRICT, ps_block=8)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=0.1, mode=STRICT, ps_block=8)
    with np.errstate(all="ignore"):
        compare_full(g, r, Q, V, causal=True, tau=0.1)
    assert g["stats"]["n_exact_tiles"] > 0


def test_attention_blocked_fullsize(dev, orc):
    """The GPT-2-XL-shaped layer (8 x 25 heads, S 1024, D 64), runs of 16,
    sampled heads against the oracle."""
    from mixed_precision_attention_ps_amd.configs import WORKLOADS, tau_for
    w = WORKLOADS["gpt2_xl_layer"]
    Q, K, V, _ = w.qkv()
    tau = tau_for(w.name, "strict", 4, 0.016)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT, want_probs=False,
                want_scores=False, ps_block=16)
    heads = [0, 123]
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT, heads=heads, ps_block=16)
    compare_full(g, r, Q, V, causal=True, tau=tau, heads=heads, check_probs=False)


DECODE_CASES = [
    # B, H, Nq, S, D, mu, tau, block
    (1, 2, 4, 500, 64, 4, 0.1, 8),
    (1, 2, 4, 500, 64, 4, 0.1, 32),
    (1, 1, 3, 300, 128, 4, 0.1, 64),
    (1, 1, 16, 400, 64, 4, 0.05, 16),
    (1, 1, 2, 300, 64, 12, 0.1, 16),     # exact double path
    (1, 1, 2, 300, 64, 23, 0.1, 8),      # mu = 23
]


@pytest.mark.parametrize("B,H,nq,S,D,mu,tau,block", DECODE_CASES)
def test_decode_blocked(dev, orc, B, H, nq, S, D, mu, tau, block):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=S + block)
    note(f"decode blocked B={B} H={H} Nq={nq} S={S} D={D} mu={mu} block={block}")
    W = (S + 31) // 32
    q = torch.from_numpy(np.ascontiguousarray(Q[:, :, S - nq:, :])).to(dev)
    k, v = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    probs = torch.zeros((B, H, nq, S), device=dev)
    mask = torch.zeros((B, H, nq, W), dtype=torch.int32, device=dev)
    kl = torch.zeros((B, H, nq), dtype=torch.float64, device=dev)
    kll = torch.zeros((B, H, nq), dtype=torch.float64, device=dev)
    cnt = torch.zeros((B, H, nq), dtype=torch.int32, device=dev)
    ymix = torch.zeros((B, H, nq, S), device=dev)
    yref = torch.zeros((B, H, nq, S), device=dev)
    out, st = lamp.lamp_decode_fwd(q, k, v, causal=True, mu=mu, tau=tau, probs=probs,
                                   recompute_mask=mask, row_kl=kl, row_kl_lowp=kll, row_count=cnt,
                                   scores_mix=ymix, scores_ref=yref, ps_block=block)
    torch.cuda.synchronize()
    g = {"out": out.cpu().numpy(), "mask": mask.cpu().numpy().view(np.uint32),
         "kl": kl.cpu().numpy(), "kl_lowp": kll.cpu().numpy(), "count": cnt.cpu().numpy(),
         "stats": st, "ymix": ymix.cpu().numpy(), "yref": yref.cpu().numpy(),
         "probs": probs.cpu().numpy()}

    class BlockedOracle:
        def lamp_heads(self, *a, **kw):
            return orc.lamp_heads(*a, ps_block=block, **kw)

    check_decode(g, BlockedOracle(), Q, K, V, nq, causal=True, mu=mu, tau=tau)


def test_decode_blocked_matches_full_relaxed_rows(dev):
    """Decode in the blocked order equals the last rows of the full relaxed
    call in the same order, bit for bit on the masks."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D, nq = 1, 2, 700, 64, 3
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=4)
    q = torch.from_numpy(np.ascontiguousarray(Q[:, :, S - nq:, :])).to(dev)
    k, v = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    W = (S + 31) // 32
    m1 = torch.zeros((B, H, nq, W), dtype=torch.int32, device=dev)
    lamp.lamp_decode_fwd(q, k, v, causal=True, mu=4, tau=0.1, recompute_mask=m1, ps_block=16)
    qf = torch.from_numpy(Q).to(dev)
    m2 = torch.zeros((B, H, S, W), dtype=torch.int32, device=dev)
    lamp.lamp_attention_fwd(qf, k, v, causal=True, mu=4, tau=0.1, mode=RELAXED,
                            recompute_mask=m2, want_stats=False, ps_block=16)
    torch.cuda.synchronize()
    assert (m1.cpu().numpy() == m2[:, :, S - nq:].cpu().numpy()).all()


MLP_CASES = [
    # op, M, N, K, mu, tau, block
    ("gelu", 70, 130, 256, 4, 0.1, 16),
    ("gelu", 33, 97, 100, 7, 0.05, 8),       # K = 100: a short last run
    ("gelu", 20, 70, 1600, 4, 0.02, 64),
    ("gelu", 31, 65, 128, 12, 0.1, 16),      # exact double path
    ("gelu", 17, 40, 64, 23, 0.1, 4),        # mu = 23
    ("gelu", 129, 200, 256, 4, 0.05, 4),     # narrow tiles
    ("gelu", 129, 200, 100, 4, 0.05, 8),     # narrow tiles, a short last run
    ("gelu", 70, 300, 256, 4, 0.05, 16),     # narrow tiles
    ("layernorm", 70, 300, 256, 4, 0.3, 16),
    ("layernorm", 9, 1600, 6400, 4, 0.3, 64),
    ("layernorm", 9, 1600, 640, 4, 0.2, 32),
    ("layernorm", 20, 70, 96, 10, 0.5, 8),
    ("layernorm", 12, 300, 6400, 4, 0.3, 256),
]


@pytest.mark.parametrize("op,M,N,K,mu,tau,block", MLP_CASES)
def test_mlp_blocked(dev, orc, op, M, N, K, mu, tau, block):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    X, W, gamma, beta = make_mlp(M, N, K, w_std=0.05, seed=M + K + block)
    note(f"{op} blocked M={M} N={N} K={K} mu={mu} tau={tau} block={block}")
    x, w, gm, bt = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (X, W, gamma, beta))
    mask = torch.zeros((M, (N + 31) // 32), dtype=torch.int32, device=dev)
    err = torch.zeros(M, dtype=torch.float64, device=dev)
    errl = torch.zeros(M, dtype=torch.float64, device=dev)
    cnt = torch.zeros(M, dtype=torch.int32, device=dev)
    ymix = torch.zeros((M, N), device=dev)
    yref = torch.zeros((M, N), device=dev)
    kw = dict(mu=mu, tau=tau, recompute_mask=mask, row_err=err, row_err_lowp=errl, row_count=cnt,
              scores_mix=ymix, scores_ref=yref, ps_block=block)
    if op == "gelu":
        out, st = lamp.lamp_gelu_fwd(x, w, **kw)
    else:
        out, st = lamp.lamp_layernorm_fwd(x, w, gm, bt, eps=1e-5, **kw)
    torch.cuda.synchronize()
    g = {"out": out.cpu().numpy(), "mask": mask.cpu().numpy().view(np.uint32),
         "err": err.cpu().numpy(), "err_lowp": errl.cpu().numpy(), "count": cnt.cpu().numpy(),
         "stats": st, "ymix": ymix.cpu().numpy(), "yref": yref.cpu().numpy()}

    class BlockedOracle:
        def ps_gemm(self, X_, W_, *, mu):
            return orc.ps_gemm(X_, W_, mu=mu, ps_block=block)

        def __getattr__(self, name):
            return getattr(orc, name)

    if op == "gelu":
        check_gelu(g, BlockedOracle(), X, W, mu=mu, tau=tau)
    else:
        _, ties = check_ln(g, BlockedOracle(), X, W, gamma, beta, mu=mu, eps=1e-5, tau=tau)
        assert ties <= 1

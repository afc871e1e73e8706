"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (mixed_precision_attention_ps_amd.inputs).
Scores, y^mix, masks and counts must match bit for bit; probabilities,
outputs and KL within the tolerances stated in tests/parity.py.
"""
import sys

import numpy as np
import pytest

from mixed_precision_attention_ps_amd.configs import WORKLOADS
from mixed_precision_attention_ps_amd.inputs import make_qkv, make_special
from tests import parity

pytestmark = pytest.mark.gpu

STRICT, RELAXED, RANDOM = 0, 1, 2
MODE_NAME = {STRICT: "strict", RELAXED: "relaxed", RANDOM: "random"}


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mixed_precision_attention_ps_amd import lamp
    lamp.library()
    return torch.device("cuda:0")


def note(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(dev, Q, K, V, *, causal, mu, tau, mode, seed=0, want_probs=True, want_mask=True,
            want_scores=True, want_rows=True, want_stats=True, ps_block=0, relaxed_path=0,
            workspace=None):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D = Q.shape
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    W = (S + 31) // 32
    probs = torch.full((B, H, S, S), -7.0, device=dev) if want_probs else None
    mask = torch.full((B, H, S, W), -1, dtype=torch.int32, device=dev) if want_mask else None
    row_kl = torch.zeros((B, H, S), dtype=torch.float64, device=dev) if want_rows else None
    row_kl_lowp = torch.zeros((B, H, S), dtype=torch.float64, device=dev) if want_rows else None
    row_count = torch.zeros((B, H, S), dtype=torch.int32, device=dev) if want_rows else None
    ymix = torch.zeros((B, H, S, S), device=dev) if want_scores else None
    yref = torch.zeros((B, H, S, S), device=dev) if want_scores else None
    note(f"gpu {MODE_NAME[mode]} B={B} H={H} S={S} D={D} causal={causal} mu={mu} tau={tau} "
         f"probs={want_probs} scores={want_scores} rows={want_rows} stats={want_stats} "
         f"ps_block={ps_block} relaxed_path={relaxed_path}")
    out, st = lamp.lamp_attention_fwd(q, k, v, causal=causal, mu=mu, tau=tau, mode=mode,
                                      probs=probs, recompute_mask=mask, seed=seed, row_kl=row_kl,
                                      row_kl_lowp=row_kl_lowp, row_count=row_count,
                                      scores_mix=ymix, scores_ref=yref, want_stats=want_stats,
                                      ps_block=ps_block, relaxed_path=relaxed_path,
                                      workspace=workspace)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy(), "stats": st}
    if want_rows:
        res.update(row_kl=row_kl.cpu().numpy(), row_kl_lowp=row_kl_lowp.cpu().numpy(),
                   row_count=row_count.cpu().numpy())
    if want_scores:
        res.update(ymix=ymix.cpu().numpy(), yref=yref.cpu().numpy())
    if want_probs:
        res["probs"] = probs.cpu().numpy()
    if want_mask:
        res["mask"] = mask.cpu().numpy().view(np.uint32)
    return res


def run_orc(orc, Q, K, V, *, causal, mu, tau, mode, seed=0, heads=None, rows=None, ps_block=0):
    note(f"oracle {MODE_NAME[mode]} shape={Q.shape} heads={heads} rows={rows} ps_block={ps_block}")
    return orc.lamp_heads(Q, K, V, causal=causal, mu=mu, tau=tau, mode=mode, seed=seed,
                          heads=heads, rows=rows, ps_block=ps_block)


def ymix_oracle(r, S):
    sel = parity.unpack_mask(r["mask"], S)
    return np.where(sel, r["yref"], r["ylo"])


def compare_full(g, r, Q, V, *, causal, tau, heads=None, rows=None, check_probs=True):
    """Compare GPU results (full [B,H,S,...]) against oracle results on the
    oracle's heads and rows."""
    B, H, S, D = Q.shape
    heads = list(range(B * H)) if heads is None else list(heads)
    rb, re_ = (0, S) if rows is None else rows
    sl = slice(rb, re_)
    valid = parity.valid_mask(S, causal, (rb, re_))[None].repeat(len(heads), 0)
    gv = lambda name: g[name].reshape((B * H,) + g[name].shape[2:])[heads][:, sl]
    if "yref" in g:
        parity.assert_bits(gv("yref"), r["yref"], valid, "FP32 reference scores")
        parity.assert_bits(gv("ymix"), ymix_oracle(r, S), valid, "mixed scores")
    ties = parity.assert_mask(gv("mask"), r["mask"], r["crit"], tau, S)
    if "row_count" in g:
        assert (gv("row_count") == r["count"]).all() or ties > 0, "row counts"
    if check_probs and "probs" in g:
        parity.assert_tol(gv("probs"), r["probs"], np.abs(r["probs"]), "probs")
    Vf = V.reshape(B * H, S, D)
    scale = np.stack([parity.out_scale(r["probs"][n].astype(np.float64), Vf[h])
                      for n, h in enumerate(heads)])
    parity.assert_tol(gv("out"), r["out"], scale, "out")
    if "row_kl" in g:
        parity.assert_tol(gv("row_kl"), r["kl"], np.abs(r["kl"]), "row KL")
        parity.assert_tol(gv("row_kl_lowp"), r["kl_lowp"], np.abs(r["kl_lowp"]), "row KL lowp")
    st = g["stats"]
    if st is not None and not heads_subset(heads, B * H, rows, S):
        assert st["n_selected"] == r["count"].sum() or ties > 0
        assert abs(st["kl_sum"] - r["kl"].sum()) <= 1e-6 * r["kl"].sum() + 1e-7 * r["kl"].size
        assert abs(st["kl_lowp_sum"] - r["kl_lowp"].sum()) <= 1e-6 * r["kl_lowp"].sum() + 1e-7 * r["kl"].size
    return ties


def heads_subset(heads, BH, rows, S):
    return len(heads) != BH or (rows is not None and tuple(rows) != (0, S))


# ---------------------------------------------------------------------------
# Step 1: scores
# ---------------------------------------------------------------------------
SCORE_CASES = [
    (1, 1, 128, 64, False, 4), (1, 2, 200, 64, True, 4), (1, 1, 1, 64, True, 4),
    (1, 1, 2, 64, False, 4), (1, 1, 63, 64, True, 4), (1, 1, 64, 64, False, 4),
    (1, 1, 65, 64, True, 4), (1, 1, 127, 64, False, 4), (2, 1, 70, 4, True, 4),
    (1, 1, 70, 8, False, 4), (1, 1, 70, 20, True, 7), (1, 1, 70, 128, True, 4),
    (1, 1, 70, 256, False, 10), (1, 1, 96, 64, True, 1), (1, 1, 96, 64, True, 2),
    (1, 1, 96, 64, True, 7), (1, 1, 96, 64, True, 10), (1, 1, 96, 64, True, 11),
    (1, 1, 96, 64, True, 16), (1, 1, 96, 64, True, 22), (1, 1, 96, 64, True, 23),
]


@pytest.mark.parametrize("B,H,S,D,causal,mu", SCORE_CASES)
def test_scores_bitexact(dev, orc, B, H, S, D, causal, mu):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=min(2, D // 4), seed=S * 7 + D + mu)
    note(f"scores B={B} H={H} S={S} D={D} causal={causal} mu={mu}")
    q, k = torch.from_numpy(Q).to(dev), torch.from_numpy(K).to(dev)
    ylo, yref = lamp.lamp_ps_scores(q, k, causal=causal, mu=mu)
    torch.cuda.synchronize()
    r = orc.lamp_heads(Q, K, V, causal=causal, mu=mu, tau=np.inf, mode=STRICT,
                       want=("ylo", "yref"))
    valid = parity.valid_mask(S, causal)[None].repeat(B * H, 0)
    parity.assert_bits(ylo.cpu().numpy().reshape(B * H, S, S), r["ylo"], valid, "PS scores")
    parity.assert_bits(yref.cpu().numpy().reshape(B * H, S, S), r["yref"], valid, "FP32 scores")


@pytest.mark.parametrize("kind", ["tiny", "huge", "mixed", "nonfinite"])
@pytest.mark.parametrize("mu", [4, 10])
def test_scores_special_values(dev, orc, kind, mu):
    """Inputs outside the fast path's operand range take the exact path."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D = 1, 2, 130, 64
    Q, K, V = make_special(B, H, S, D, kind=kind, seed=mu)
    note(f"special scores kind={kind} mu={mu}")
    q, k = torch.from_numpy(Q).to(dev), torch.from_numpy(K).to(dev)
    ylo, yref = lamp.lamp_ps_scores(q, k, causal=True, mu=mu)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        r = orc.lamp_heads(Q, K, V, causal=True, mu=mu, tau=np.inf, mode=STRICT,
                           want=("ylo", "yref"))
    valid = parity.valid_mask(S, True)[None].repeat(B * H, 0)
    parity.assert_bits(ylo.cpu().numpy().reshape(B * H, S, S), r["ylo"], valid, "PS scores")
    parity.assert_bits(yref.cpu().numpy().reshape(B * H, S, S), r["yref"], valid, "FP32 scores")


# ---------------------------------------------------------------------------
# The whole strict / random path
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [1e-1, 1e-2, 1e-3])
def test_strict_single_head(dev, orc, tau):
    w = WORKLOADS["single_head_s128"]
    Q, K, V, _ = w.qkv()
    g = run_gpu(dev, Q, K, V, causal=False, mu=4, tau=tau, mode=STRICT)
    r = run_orc(orc, Q, K, V, causal=False, mu=4, tau=tau, mode=STRICT)
    ties = compare_full(g, r, Q, V, causal=False, tau=tau)
    assert ties == 0
    st = g["stats"]
    assert st["n_selected"] == r["count"].sum() and st["n_valid"] == 128 * 128
    assert abs(st["kl_sum"] - r["kl"].sum()) <= 1e-6 * r["kl"].sum() + 1e-7


@pytest.fixture(scope="module")
def gpt2_small():
    return WORKLOADS["gpt2_small_s1024"].qkv()[:3]


@pytest.mark.parametrize("tau", [1e-1, 1e-2, 1e-3, 1e-4])
def test_strict_gpt2_small(dev, orc, gpt2_small, tau):
    Q, K, V = gpt2_small
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    compare_full(g, r, Q, V, causal=True, tau=tau)
    assert g["stats"]["n_selected"] == r["count"].sum()


def test_random_control_gpt2_small(dev, orc, gpt2_small):
    Q, K, V = gpt2_small
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RANDOM, seed=1234)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RANDOM, seed=1234)
    S = Q.shape[2]
    gm = g["mask"].reshape(-1, S, (S + 31) // 32)
    assert (gm == r["mask"]).all(), "random-control masks"
    compare_full(g, r, Q, V, causal=True, tau=np.inf)
    # the adaptive selection beats the random one at the same per-row counts
    st = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    assert (st["row_count"] == g["row_count"]).all()
    assert st["row_kl"].mean() <= g["row_kl"].mean() / 2


@pytest.mark.parametrize("tau", [0.0, np.inf])
def test_tau_limits(dev, orc, tau):
    Q, K, V, _ = make_qkv(1, 2, 160, 64, n_outlier=2, seed=21)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    compare_full(g, r, Q, V, causal=True, tau=tau)
    if np.isinf(tau):
        assert g["row_count"].sum() == 0
        # two kernels sum the same terms in different orders
        np.testing.assert_allclose(g["row_kl"], g["row_kl_lowp"], rtol=1e-10, atol=1e-14)


def test_strict_special_inputs(dev, orc):
    """Zeros, tiny and huge operands in the full path (exact-path tiles)."""
    Q, K, V = make_special(1, 2, 150, 64, kind="mixed", seed=3)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=STRICT)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=1e-2, mode=STRICT)
    compare_full(g, r, Q, V, causal=True, tau=1e-2)
    assert g["stats"]["n_exact_tiles"] > 0


def test_determinism(dev, gpt2_small):
    Q, K, V = gpt2_small
    a = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=STRICT)
    b = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=STRICT)
    for name in ("mask", "ymix", "yref", "row_count", "probs", "out", "row_kl"):
        assert np.array_equal(a[name].view(np.uint8), b[name].view(np.uint8)), name


# ---------------------------------------------------------------------------
# Relaxed one-pass path
# ---------------------------------------------------------------------------
RELAXED_CASES = [
    (1, 2, 256, 64, True, 4, 1e-2), (1, 1, 200, 64, False, 4, 1e-2),
    (1, 1, 130, 128, True, 4, 1e-2), (1, 1, 100, 64, True, 23, 1e-3),
    (1, 1, 100, 64, True, 11, 1e-3), (1, 1, 1, 64, True, 4, 0.0), (1, 1, 70, 8, False, 7, 1e-1),
]


# relaxed_path 1: the fused one-pass kernel (online softmax); 2: the score
# tiles, then the row pass with the relaxed rule (rows of <= 1024 keys)
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("B,H,S,D,causal,mu,tau", RELAXED_CASES)
def test_relaxed_small(dev, orc, B, H, S, D, causal, mu, tau, path):
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=min(2, D // 4), seed=S + D)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=mu, tau=tau, mode=RELAXED, relaxed_path=path)
    r = run_orc(orc, Q, K, V, causal=causal, mu=mu, tau=tau, mode=RELAXED)
    compare_full(g, r, Q, V, causal=causal, tau=tau)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("kind", ["mixed", "tiny"])
def test_relaxed_special_inputs(dev, orc, kind, path):
    """Out-of-range operands (exact-path tiles); in "mixed" a few huge
    operands give rows whose maximum lies far above earlier blocks' maxima
    (exp(m - m_t) overflows: the relaxed row pass takes exp(y - m_t)
    directly)."""
    Q, K, V = make_special(1, 1, 140, 64, kind=kind, seed=9)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=RELAXED, relaxed_path=path)
    with np.errstate(all="ignore"):
        r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=1e-2, mode=RELAXED)
    compare_full(g, r, Q, V, causal=True, tau=1e-2)
    assert g["stats"]["n_exact_tiles"] > 0


@pytest.mark.parametrize("tau", [0.0, 1e-3])
def test_relaxed_paths_agree(dev, orc, gpt2_small, tau):
    """The two relaxed implementations select the same keys and form the
    same y^mix bit for bit; each matches the oracle."""
    Q, K, V = gpt2_small
    a = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=1)
    b = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=2)
    for name in ("mask", "ymix", "yref", "row_count"):
        assert np.array_equal(a[name].view(np.uint8), b[name].view(np.uint8)), name
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, heads=[0, 11])
    for g in (a, b):
        compare_full(g, r, Q, V, causal=True, tau=tau, heads=[0, 11])


@pytest.mark.parametrize("path", [1, 2])
def test_relaxed_superset_of_strict(dev, gpt2_small, path):
    Q, K, V = gpt2_small
    st = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=STRICT)
    rl = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=RELAXED, relaxed_path=path)
    S = Q.shape[2]
    a = parity.unpack_mask(st["mask"], S)
    b = parity.unpack_mask(rl["mask"], S)
    assert not (a & ~b).any()


def test_device_exponentials_accuracy(dev):
    """The double exp (criterion, KL sums) and the FP32-accurate exp
    (probabilities) against the host's libm exp."""
    import math

    import torch
    from mixed_precision_attention_ps_amd import lamp
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-745, 709, 20000), rng.uniform(-40, 0, 20000),
                        rng.uniform(-1, 1, 5000), [0.0, -1e-300, 1e-300, -700.0, 700.0]])
    y64, y32 = lamp.lamp_diag_exp(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    y64, y32 = y64.cpu().numpy(), y32.cpu().numpy()
    ref = np.array([math.exp(v) for v in x])
    normal = ref > 1e-300
    rel64 = np.abs(y64[normal] - ref[normal]) / ref[normal]
    assert rel64.max() < 1e-15, rel64.max()
    f32 = (x > -87) & (x < 88)
    rel32 = np.abs(y32[f32].astype(np.float64) - ref[f32]) / ref[f32]
    assert rel32.max() < 4e-7, rel32.max()
    assert (y32[x < -110] == 0).all()


# Which optional buffers the caller passes decides where the strict path keeps
# y^lo / y^mix / probabilities (in place or in the workspace): every
# combination against the oracle.
@pytest.mark.parametrize("probs,scores,rows,stats", [
    (True, False, True, False), (False, False, True, False), (True, True, False, True),
    (False, True, True, True), (False, False, False, True), (True, False, False, False)])
def test_strict_buffer_configurations(dev, orc, probs, scores, rows, stats):
    Q, K, V, _ = make_qkv(1, 3, 320, 64, n_outlier=2, seed=77)
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT, want_probs=probs,
                want_scores=scores, want_rows=rows, want_stats=stats)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    compare_full(g, r, Q, V, causal=True, tau=tau)


@pytest.mark.parametrize("S,causal,mode", [(1100, True, STRICT), (1300, False, STRICT),
                                           (1025, True, RANDOM), (2048, True, RELAXED)])
def test_rows_longer_than_1024(dev, orc, S, causal, mode):
    """Rows past 1024 keys take the streaming (multi-kernel) strict path."""
    Q, K, V, _ = make_qkv(1, 1, S, 64, n_outlier=2, seed=S)
    tau = 1e-2
    rows = (S - 80, S)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=4, tau=tau, mode=mode, seed=5)
    r = run_orc(orc, Q, K, V, causal=causal, mu=4, tau=tau, mode=mode, seed=5, rows=rows)
    compare_full(g, r, Q, V, causal=causal, tau=tau, rows=rows)
    r0 = run_orc(orc, Q, K, V, causal=causal, mu=4, tau=tau, mode=mode, seed=5, rows=(0, 64))
    compare_full(g, r0, Q, V, causal=causal, tau=tau, rows=(0, 64))


# ---------------------------------------------------------------------------
# Relaxed rule over rows longer than 1024 keys in two passes (relaxed_path 2:
# score tiles with partials, one streaming row pass, softmax and P.V)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,causal,D,tau", [(1100, True, 64, 1e-2), (1300, False, 64, 1e-3),
                                            (1025, True, 128, 1e-2), (1090, True, 64, 0.0)])
def test_relaxed_long_rows_two_pass(dev, orc, S, causal, D, tau):
    Q, K, V, _ = make_qkv(1, 2, S, D, n_outlier=2, seed=S + D)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=4, tau=tau, mode=RELAXED, relaxed_path=2)
    for rows in ((0, 64), (S // 2 - 20, S // 2 + 20), (S - 70, S)):
        r = run_orc(orc, Q, K, V, causal=causal, mu=4, tau=tau, mode=RELAXED, rows=rows)
        compare_full(g, r, Q, V, causal=causal, tau=tau, rows=rows)


@pytest.mark.parametrize("tau", [0.0, 1e-2])
def test_relaxed_long_rows_paths_agree(dev, orc, tau):
    """Fused one-pass kernel and two passes on rows of 1100 keys: the same
    masks, counts and y^mix bit for bit."""
    Q, K, V, _ = make_qkv(1, 3, 1100, 64, n_outlier=2, seed=41)
    a = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=1)
    b = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=2)
    for name in ("mask", "ymix", "yref", "row_count"):
        assert np.array_equal(a[name].view(np.uint8), b[name].view(np.uint8)), name
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, heads=[1],
                rows=(1000, 1100))
    for g in (a, b):
        compare_full(g, r, Q, V, causal=True, tau=tau, heads=[1], rows=(1000, 1100))


@pytest.mark.parametrize("kind", ["mixed", "tiny"])
def test_relaxed_long_rows_special_inputs(dev, orc, kind):
    """Out-of-range operands (exact-path tiles, with their partials) in rows
    longer than 1024 keys; in "mixed" some rows' maxima lie far above the
    earlier blocks' maxima."""
    Q, K, V = make_special(1, 1, 1100, 64, kind=kind, seed=9)
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=1e-2, mode=RELAXED, relaxed_path=2)
    for rows in ((0, 64), (1040, 1100)):
        with np.errstate(all="ignore"):
            r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=1e-2, mode=RELAXED, rows=rows)
        compare_full(g, r, Q, V, causal=True, tau=1e-2, rows=rows)
    assert g["stats"]["n_exact_tiles"] > 0


# Where y^lo / y^mix live (probabilities buffer, the caller's score buffer or
# the workspace) and which optional outputs are written, on the long-row
# two-pass path.
@pytest.mark.parametrize("probs,scores,rows,stats", [
    (True, False, True, False), (False, False, True, False), (True, True, False, True),
    (False, True, True, True), (False, False, False, True)])
def test_relaxed_long_rows_buffer_configurations(dev, orc, probs, scores, rows, stats):
    Q, K, V, _ = make_qkv(1, 1, 1088, 64, n_outlier=2, seed=78)
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, want_probs=probs,
                want_scores=scores, want_rows=rows, want_stats=stats, relaxed_path=2)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, rows=(1024, 1088))
    compare_full(g, r, Q, V, causal=True, tau=tau, rows=(1024, 1088))


def test_relaxed_long_rows_default_fits_the_workspace(dev, orc):
    """relaxed_path 0 on rows longer than 1024 keys: with a caller workspace
    that holds the fused kernel's per-row state but not the two-pass score
    buffers, the fused kernel runs; with the two-pass size, two passes run
    (each run's output equals, bit for bit, that of the implementation named
    explicitly; the two implementations round the output differently).  All
    give the oracle's masks and y^mix."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D = 1, 2, 1100, 64
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=43)
    tau = 1e-2

    def size(rp):
        p = lamp.LampParams()
        p.relaxed_path = rp
        p.row_kl = p.row_kl_lowp = p.row_count = 256   # passed by the caller (non-NULL)
        p.scores_mix = p.scores_ref = 256
        return lamp.lamp_workspace_bytes_ex(B, H, S, D, 1, "relaxed", 1, 1, p)

    small, large = size(1), size(0)
    assert 0 < small < large
    fused = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=1)
    two = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=2)
    assert not np.array_equal(fused["out"], two["out"])
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, rows=(S - 60, S))
    for nbytes, want in ((small, fused), (large, two)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, workspace=ws)
        assert np.array_equal(g["out"].view(np.uint32), want["out"].view(np.uint32))
        compare_full(g, r, Q, V, causal=True, tau=tau, rows=(S - 60, S))
        del ws


# lamp_workspace_bytes_ex is exact: a call runs in that many bytes (with the
# same results as with the library's pool) and is refused with 256 fewer,
# except where the relaxed default falls back to the fused kernel.
@pytest.mark.parametrize("mode", [STRICT, RELAXED, RANDOM])
@pytest.mark.parametrize("S", [300, 1100])
@pytest.mark.parametrize("probs", [True, False])
def test_workspace_bytes_ex_is_exact(dev, mode, S, probs):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, D = 1, 2, 64
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=S + mode)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    need = lamp.lamp_workspace_bytes_ex(B, H, S, D, 1, mode, int(probs), 1, None)
    assert need > 0

    def call(ws):
        p = torch.zeros((B, H, S, S), device=dev) if probs else None
        out, st = lamp.lamp_attention_fwd(q, k, v, causal=True, mu=4, tau=1e-2, mode=mode,
                                          probs=p, want_stats=True, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), st

    note(f"workspace exact mode={MODE_NAME[mode]} S={S} probs={probs} need={need}")
    ref_out, ref_st = call(None)
    buf = torch.empty(need + 4096, dtype=torch.uint8, device=dev)
    out, st = call(buf[:need])
    assert np.array_equal(out.view(np.uint32), ref_out.view(np.uint32))
    assert st["n_selected"] == ref_st["n_selected"]
    falls_back = mode == RELAXED and S > 1024
    if falls_back:   # the fused one-pass kernel runs in the smaller workspace
        out2, st2 = call(buf[:need - 256])
        assert st2["n_selected"] == ref_st["n_selected"]
    else:
        with pytest.raises(lamp.LampError):
            call(buf[:need - 256])
    del buf


# Without a KL request the score tiles' partials carry only the maxima (no
# reference sums); the relaxed two-pass forms must give the same masks,
# y^mix, probabilities and outputs, bit for bit, as with the KL.
@pytest.mark.parametrize("S", [320, 1100])
def test_relaxed_two_pass_without_kl(dev, orc, S):
    Q, K, V, _ = make_qkv(1, 2, S, 64, n_outlier=2, seed=S + 5)
    tau = 1e-2
    with_kl = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=2)
    no_kl = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, relaxed_path=2,
                    want_rows=False, want_stats=False)
    for name in ("mask", "ymix", "yref", "probs", "out"):
        assert np.array_equal(with_kl[name].view(np.uint8), no_kl[name].view(np.uint8)), name
    rows = (S - 64, S)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=RELAXED, rows=rows)
    compare_full(no_kl, r, Q, V, causal=True, tau=tau, rows=rows)

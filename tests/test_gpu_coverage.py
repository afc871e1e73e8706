"""GPU parity over whole tensors and over the paths the other suites leave
thin, against the oracle (bars of tests/parity.py):

  * the GPT-2-XL-shaped layer (8x25x1024x64, causal, mu = 4, tau for ~1.6 %
    recompute), every one of its 200 heads and 1024 rows:
      - in the benchmark's configuration (probabilities, mask and row KL
        written): masks and counts bit-exact, probabilities, out and both row
        KLs within tolerance;
      - with the score buffers passed too: y^ref and y^mix bit-exact;
      - in the serving configuration (no row KL, no statistics, no score
        buffers): the selected scores' FP32 values come from the gather dot;
  * the S = 4096 layer (4x25x4096x64): all 100 heads on sampled rows, strict
    and relaxed;
  * the gather FP32 recompute of the fused row pass at D = 64, 128 and at a
    head dimension only known at run time (D = 96), and on operands outside
    the fast path's range;
  * rows longer than 1024 keys without a row KL: no dense y^ref (the
    workspace shrinks by one score buffer), the recompute forms each selected
    key's dot from the gathered query and key rows.
"""
import gc
import sys

import numpy as np
import pytest

from mixed_precision_attention_ps_amd.configs import WORKLOADS, tau_for
from mixed_precision_attention_ps_amd.inputs import make_qkv, make_special
from tests import parity
from tests.test_gpu_parity import RANDOM, RELAXED, STRICT, compare_full, run_gpu, run_orc

pytestmark = pytest.mark.gpu


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


XL = "gpt2_xl_layer"
HEAD_CHUNK = 25   # heads the oracle evaluates (and the host compares) at a time


@pytest.fixture(scope="module")
def xl_inputs():
    return WORKLOADS[XL].qkv()[:3]


def xl_call(dev, Q, K, V, *, tau, kl, scores, stats, mode=STRICT):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D = Q.shape
    W = (S + 31) // 32
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    t = {"probs": torch.full((B, H, S, S), -7.0, device=dev),
         "mask": torch.full((B, H, S, W), -1, dtype=torch.int32, device=dev)}
    if kl:
        t["row_kl"] = torch.zeros((B, H, S), dtype=torch.float64, device=dev)
        t["row_kl_lowp"] = torch.zeros((B, H, S), dtype=torch.float64, device=dev)
        t["row_count"] = torch.zeros((B, H, S), dtype=torch.int32, device=dev)
    if scores:
        t["scores_mix"] = torch.zeros((B, H, S, S), device=dev)
        t["scores_ref"] = torch.zeros((B, H, S, S), device=dev)
    note(f"full tensor {XL} mode={mode} tau={tau} kl={kl} scores={scores} stats={stats}")
    out, st = lamp.lamp_attention_fwd(q, k, v, causal=True, mu=4, tau=tau, mode=mode,
                                      probs=t["probs"], recompute_mask=t["mask"],
                                      row_kl=t.get("row_kl"), row_kl_lowp=t.get("row_kl_lowp"),
                                      row_count=t.get("row_count"),
                                      scores_mix=t.get("scores_mix"),
                                      scores_ref=t.get("scores_ref"), want_stats=stats)
    torch.cuda.synchronize()
    t["out"] = out
    return t, st


def compare_chunked(orc, t, st, Q, K, V, tau, *, kl, scores, mode=STRICT):
    """Every head against the oracle, HEAD_CHUNK heads at a time."""
    B, H, S, D = Q.shape
    BH = B * H
    valid = parity.valid_mask(S, True)
    Vf = V.reshape(BH, S, D)
    count_sum, kl_sum, ties = 0, 0.0, 0
    for h0 in range(0, BH, HEAD_CHUNK):
        heads = list(range(h0, min(BH, h0 + HEAD_CHUNK)))
        sl = slice(h0, heads[-1] + 1)
        want = ["crit", "mask", "probs", "out", "kl", "kl_lowp", "count"]
        if scores:
            want += ["ylo", "yref"]
        r = orc.lamp_heads(Q, K, V, causal=True, mu=4, tau=tau, mode=mode, heads=heads,
                           want=tuple(want))
        g = lambda name, shape: t[name].view(BH, *shape)[sl].cpu().numpy()
        ties += parity.assert_mask(g("mask", (S, (S + 31) // 32)).view(np.uint32), r["mask"],
                                   r["crit"], tau, S)
        parity.assert_tol(g("probs", (S, S)), r["probs"], np.abs(r["probs"]), "probs")
        scale = np.stack([parity.out_scale(r["probs"][n].astype(np.float64), Vf[h])
                          for n, h in enumerate(heads)])
        parity.assert_tol(g("out", (S, D)), r["out"], scale, "out")
        if kl:
            assert (g("row_count", (S,)) == r["count"]).all() or ties > 0, "row counts"
            parity.assert_tol(g("row_kl", (S,)), r["kl"], np.abs(r["kl"]), "row KL")
            parity.assert_tol(g("row_kl_lowp", (S,)), r["kl_lowp"], np.abs(r["kl_lowp"]),
                              "row KL lowp")
        if scores:
            vm = np.broadcast_to(valid, (len(heads), S, S))
            parity.assert_bits(g("scores_ref", (S, S)), r["yref"], vm, "FP32 reference scores")
            sel = parity.unpack_mask(r["mask"], S)
            parity.assert_bits(g("scores_mix", (S, S)), np.where(sel, r["yref"], r["ylo"]), vm,
                               "mixed scores")
        count_sum += int(r["count"].sum())
        kl_sum += float(r["kl"].sum())
        del r
        gc.collect()
    assert ties == 0
    if st is not None:
        assert st["n_selected"] == count_sum
        assert abs(st["kl_sum"] - kl_sum) <= 1e-6 * kl_sum + 1e-7 * BH * S
        assert st["n_valid"] == WORKLOADS[XL].n_valid


def test_xl_full_tensor_bench_configuration(dev, orc, xl_inputs):
    Q, K, V = xl_inputs
    tau = tau_for(XL, "strict", 4, 0.016)
    t, st = xl_call(dev, Q, K, V, tau=tau, kl=True, scores=False, stats=True)
    compare_chunked(orc, t, st, Q, K, V, tau, kl=True, scores=False)


def test_xl_full_tensor_scores(dev, orc, xl_inputs):
    Q, K, V = xl_inputs
    tau = tau_for(XL, "strict", 4, 0.016)
    t, st = xl_call(dev, Q, K, V, tau=tau, kl=True, scores=True, stats=False)
    compare_chunked(orc, t, None, Q, K, V, tau, kl=True, scores=True)


def test_xl_full_tensor_serving_gather(dev, orc, xl_inputs):
    """No row KL, no statistics and no score buffers: the score tiles keep no
    y^ref and the fused row pass forms every selected score's FP32 dot."""
    Q, K, V = xl_inputs
    tau = tau_for(XL, "strict", 4, 0.016)
    t, st = xl_call(dev, Q, K, V, tau=tau, kl=False, scores=False, stats=False)
    compare_chunked(orc, t, None, Q, K, V, tau, kl=False, scores=False)


def test_xl_full_tensor_relaxed_bench_configuration(dev, orc, xl_inputs):
    """The relaxed rule in the bench's configuration (the library's choice:
    score tiles, then the relaxed row pass with P.V; probabilities, mask, row
    KLs and statistics), every head and row against the oracle."""
    from mixed_precision_attention_ps_amd import lamp
    Q, K, V = xl_inputs
    tau = tau_for(XL, "relaxed", 4, 0.016)
    t, st = xl_call(dev, Q, K, V, tau=tau, kl=True, scores=False, stats=True, mode=RELAXED)
    assert lamp.IMPLS[st["impl"]] == "relaxed_rows"
    compare_chunked(orc, t, st, Q, K, V, tau, kl=True, scores=False, mode=RELAXED)


R4K = "relaxed_s4096"
R4K_ROWS = [(0, 40), (2040, 2080), (4056, 4096)]


@pytest.mark.parametrize("mode,tau", [(STRICT, 1e-2), (RELAXED, 1e-2)])
def test_s4096_all_heads_sampled_rows(dev, orc, mode, tau):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    w = WORKLOADS[R4K]
    Q, K, V = w.qkv()[:3]
    B, H, S, D = Q.shape
    BH, W = B * H, (S + 31) // 32
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    probs = torch.full((B, H, S, S), -7.0, device=dev)
    mask = torch.full((B, H, S, W), -1, dtype=torch.int32, device=dev)
    row_kl = torch.zeros((B, H, S), dtype=torch.float64, device=dev)
    row_count = torch.zeros((B, H, S), dtype=torch.int32, device=dev)
    note(f"{R4K} all heads mode={mode} tau={tau}")
    out, st = lamp.lamp_attention_fwd(q, k, v, causal=True, mu=4, tau=tau, mode=mode, probs=probs,
                                      recompute_mask=mask, row_kl=row_kl, row_count=row_count,
                                      want_stats=True)
    torch.cuda.synchronize()
    assert st["n_valid"] == w.n_valid
    heads = list(range(BH))
    Vf = V.reshape(BH, S, D)
    for rb, re_ in R4K_ROWS:
        note(f"oracle {R4K} all heads rows={rb}..{re_}")
        r = orc.lamp_heads(Q, K, V, causal=True, mu=4, tau=tau, mode=mode, heads=heads,
                           rows=(rb, re_), want=("crit", "mask", "probs", "out", "kl", "count"))
        ties = parity.assert_mask(mask.view(BH, S, W)[:, rb:re_].cpu().numpy().view(np.uint32),
                                  r["mask"], r["crit"], tau, S)
        assert ties == 0
        assert (row_count.view(BH, S)[:, rb:re_].cpu().numpy() == r["count"]).all()
        parity.assert_tol(probs.view(BH, S, S)[:, rb:re_].cpu().numpy(), r["probs"],
                          np.abs(r["probs"]), "probs")
        scale = np.stack([parity.out_scale(r["probs"][h].astype(np.float64), Vf[h])
                          for h in heads])
        parity.assert_tol(out.view(BH, S, D)[:, rb:re_].cpu().numpy(), r["out"], scale, "out")
        parity.assert_tol(row_kl.view(BH, S)[:, rb:re_].cpu().numpy(), r["kl"], np.abs(r["kl"]),
                          "row KL")
        del r
        gc.collect()
    del q, k, v, probs, mask, row_kl, row_count, out
    gc.collect()
    torch.cuda.empty_cache()


# The fused row pass's gather FP32 recompute (strict, no row KL and no
# scores_ref: the score tiles keep no y^ref) at the compile-time head
# dimensions and at one only known at run time.  The relaxed row pass keeps
# y^ref for its partials; its cases here check the same shapes without row
# outputs.
@pytest.mark.parametrize("D", [64, 128, 96])
@pytest.mark.parametrize("mode", [STRICT, RELAXED])
def test_fused_no_row_outputs(dev, orc, D, mode):
    Q, K, V, _ = make_qkv(1, 3, 320, D, n_outlier=2, seed=D + mode)
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=mode, want_scores=False,
                want_rows=False, want_stats=False, relaxed_path=2)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=mode)
    compare_full(g, r, Q, V, causal=True, tau=tau)


@pytest.mark.parametrize("kind", ["mixed", "tiny"])
def test_fused_gather_special_inputs(dev, orc, kind):
    """Zeros, tiny and huge operands (exact-path score tiles) with the gather
    dot: the selected scores' FP32 values must equal the oracle's sequential
    FP32 dot bit for bit (checked through y^mix in a second call with the
    score buffers, which takes them from the tiles instead)."""
    Q, K, V = make_special(1, 2, 150, 64, kind=kind, seed=11)
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT, want_scores=False,
                want_rows=False, want_stats=False)
    with np.errstate(all="ignore"):
        r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    compare_full(g, r, Q, V, causal=True, tau=tau)
    h = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=STRICT)
    for name in ("mask", "probs", "out"):
        assert np.array_equal(g[name].view(np.uint8), h[name].view(np.uint8)), name


# Rows longer than 1024 keys without a row KL: no dense y^ref in the
# workspace; the recompute forms the selected keys' dots from the gathered
# rows.
@pytest.mark.parametrize("S,causal,D,mode", [(1100, True, 64, STRICT), (1300, False, 64, STRICT),
                                             (1030, True, 128, STRICT), (1025, True, 64, RANDOM),
                                             (1090, True, 96, STRICT)])
def test_long_rows_gather_recompute(dev, orc, S, causal, D, mode):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H = 1, 2
    with_kl = lamp.lamp_workspace_bytes_ex(B, H, S, D, int(causal), mode, 1, 1, None)
    without = lamp.lamp_workspace_bytes_ex(B, H, S, D, int(causal), mode, 1, 0, None)
    assert without <= with_kl - 4 * B * H * S * S   # y^ref is not kept
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=S + D)
    tau = 1e-2
    ws = torch.empty(without, dtype=torch.uint8, device=dev)
    g = run_gpu(dev, Q, K, V, causal=causal, mu=4, tau=tau, mode=mode, seed=9,
                want_scores=False, want_rows=False, want_stats=False, workspace=ws)
    for rows in ((0, 64), (S - 70, S)):
        r = run_orc(orc, Q, K, V, causal=causal, mu=4, tau=tau, mode=mode, seed=9, rows=rows)
        if mode == RANDOM:
            assert (g["mask"].reshape(B * H, S, -1)[:, rows[0]:rows[1]] == r["mask"]).all()
        compare_full(g, r, Q, V, causal=causal, tau=np.inf if mode == RANDOM else tau, rows=rows)


# Head orders: with the heads a multiple of 8 the score tiles take one head
# after another per XCD, and the fused row kernel walks batches of heads per
# XCD (the largest divisor of an XCD's head count up to 5: 3 at 24 heads, 2 at
# 16): every (head, row group) must still be computed once, against the oracle
# on every head.
@pytest.mark.parametrize("B,H,S,mode", [(3, 8, 320, STRICT), (2, 8, 200, RELAXED),
                                        (1, 16, 130, STRICT), (1, 40, 96, STRICT)])
def test_head_orders(dev, orc, B, H, S, mode):
    Q, K, V, _ = make_qkv(B, H, S, 64, n_outlier=2, seed=B * 100 + H)
    tau = 1e-2
    g = run_gpu(dev, Q, K, V, causal=True, mu=4, tau=tau, mode=mode, relaxed_path=2)
    r = run_orc(orc, Q, K, V, causal=True, mu=4, tau=tau, mode=mode)
    compare_full(g, r, Q, V, causal=True, tau=tau)

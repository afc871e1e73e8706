#!/usr/bin/env python3
"""Benchmark: LAMP attention forward on one MI355X.

One step = one lamp_attention_fwd call over the whole hot path (PS(mu) and
FP32 score tiles, look-ahead selection + compaction, gather FP32 recompute,
softmax + P.V + row KL), inputs resident in HBM, outputs preallocated, probs,
recompute mask and row KL written.  Default workload: the GPT-2-XL-shaped
layer (B=8, H=25, S=1024, D=64, causal, 2 outlier channels x8), strict LAMP,
mu=4, tau calibrated on the oracle to ~1.6% recompute.

Prints one JSON line with throughput (valid query-key scores per second),
the dominant kernel's ALU roofline (achieved vs peak lane-operation rate,
timed live with HIP events around that kernel's stage), and the CPU oracle
timed on this host on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode strict|relaxed|random]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LAMP attention scores/sec at μ=4 (GPT-2-XL layer) + % VALU/HBM roofline"

# MI355X 32-bit VALU peak in lane-operations per second: the published FP32
# vector rate, 157.3 TFLOP/s, counts 2 flops per FMA lane-operation, i.e.
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 7.86e13 lane-operations/s.  (The
# score kernel's measured 9-instruction MAC sequence runs above the 16-lane
# figure, 3.9e13/s, so 32-bit ALU instructions do issue at this rate.)
ALU_PEAK = 256 * 4 * 32 * 2.4e9
HBM_PEAK = 8.0e12

# The sources each measured kernel is built from (its traffic entry is stale
# once any of them changes).
_COMMON = ["lamp_device.h", "lamp_exp.h", "lamp_internal.h"]
KERNEL_SOURCES = {
    "ps_scores_kernel": _COMMON + ["scores.hip"],
    "relaxed_kernel": _COMMON + ["relaxed.hip"],
    "decode_scores_kernel": _COMMON + ["decode.hip"],
    "decode_softmax_kernel": _COMMON + ["decode.hip"],
    "ps_gemm_kernel": _COMMON + ["mlp.hip"],
}


def run_flush_ops(n: int, block: int) -> int:
    """Lane-operations the blocked PS(mu) order adds to an n-term dot: one
    PS(mu) add (add + 3-instruction rounding) per run of `block` products."""
    if block <= 1 or block >= n:
        return 0
    return 4 * ((n + block - 1) // block)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "mixed_precision_attention_ps_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(f"{kernel}/{workload}")
    if not ent or ent.get("source_sha") != kernel_source_sha(kernel):
        return None
    return ent.get("bytes_per_launch")


CPU_TARGET_S = 10.0   # wall time the oracle sample should take


def cpu_baseline(Q, K, V, w, mode_id, mu, tau, seed, ps_block=0):
    """The oracle on whole heads of the workload, spread over the layer, until
    about CPU_TARGET_S seconds have passed (or every head is done)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    BH = w.B * w.H
    order = [int(x) for x in np.random.default_rng(0).permutation(BH)]
    threads = oracle.max_threads()
    per_head = w.S * (w.S + 1) // 2 if w.causal else w.S * w.S
    done, dt = 0, 0.0
    while done < BH and dt < CPU_TARGET_S:
        heads = order[done:done + 8]
        t0 = time.perf_counter()
        oracle.lamp_heads(Q, K, V, causal=w.causal, mu=mu, tau=tau, mode=mode_id, heads=heads,
                          seed=seed, ps_block=ps_block,
                          want=("out", "kl", "count", "mask", "probs"))
        dt += time.perf_counter() - t0
        done += len(heads)
    n = per_head * done
    return {"value": n / dt, "unit": "scores/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {BH} heads (all rows, heads in a seeded random order) of "
                      f"{w.name}, same mu/tau/mode; {n} valid scores in {dt:.2f} s wall, "
                      f"{threads} OpenMP threads"}


def tau_for_workload(name: str, mode: str, mu: int, rate: float) -> float:
    from mixed_precision_attention_ps_amd.configs import tau_for
    return tau_for(name, mode, mu, rate)


def copy_calibration(args, dev):
    """A plain device copy of known size (the scale of the HBM counters), and
    a read-only reduction over the same bytes (a cross-check of the read
    scale)."""
    import torch
    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a
        s = torch.amax(b)
        torch.cuda.synchronize()
        del b, s


def decode_cpu_baseline(Q, K, V, w, nq, mu, tau, ps_block=0):
    import numpy as np
    import oracle
    oracle.build(force=False)
    BH = w.B * w.H
    order = [int(x) for x in np.random.default_rng(0).permutation(BH)]
    threads = oracle.max_threads()
    S = w.S
    per_head = sum((S - nq + t + 1) if w.causal else S for t in range(nq))
    done, dt = 0, 0.0
    while done < BH and dt < CPU_TARGET_S:
        heads = order[done:done + 8]
        t0 = time.perf_counter()
        oracle.lamp_heads(Q, K, V, causal=w.causal, mu=mu, tau=tau, mode=oracle.RELAXED,
                          heads=heads, rows=(S - nq, S), ps_block=ps_block,
                          want=("out", "kl", "count", "mask", "probs"))
        dt += time.perf_counter() - t0
        done += len(heads)
    n = per_head * done
    return {"value": n / dt, "unit": "scores/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {BH} heads, their {nq} decode rows, of {w.name}; "
                      f"{n} valid scores in {dt:.2f} s wall, {threads} OpenMP threads"}


def bench_decode(args, w):
    """Relaxed LAMP at decode shapes (lamp_decode_fwd): Nq queries per head
    against the workload's key cache.  HBM-bound at small Nq: the dominant
    kernel is reported against the HBM peak, with algorithmic bytes = the
    K (score pass) or V (softmax pass) cache read once plus the score
    buffers that pass moves."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    from mixed_precision_attention_ps_amd.configs import tau_for
    nq = args.nq
    tau = args.tau if args.tau is not None else tau_for(w.name, "relaxed", args.mu, args.rate)
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name} decode nq={nq} mu={args.mu} tau={tau}")
    Q, K, V, _ = w.qkv()
    B, H, S, D = w.B, w.H, w.S, w.D
    q = torch.from_numpy(np.ascontiguousarray(Q[:, :, S - nq:, :])).to(dev)
    k, v = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    out = torch.empty_like(q)
    probs = None if args.no_probs else torch.empty((B, H, nq, S), device=dev)
    mask = torch.empty((B, H, nq, (S + 31) // 32), dtype=torch.int32, device=dev)
    row_kl = torch.empty((B, H, nq), dtype=torch.float64, device=dev)
    copy_calibration(args, dev)

    def step(events=None):
        lamp.lamp_decode_fwd(q, k, v, causal=w.causal, mu=args.mu, tau=tau, out=out, probs=probs,
                             recompute_mask=mask, row_kl=row_kl, want_stats=False,
                             stage_events=events, ps_block=args.ps_block)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [lamp.HipEvents(2 * lamp.LAMP_N_STAGES) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(ev[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = {}
    for name in ("scores", "select", "finish"):
        si = lamp.STAGES.index(name)
        stages[name] = sum(e.elapsed_ms(2 * si, 2 * si + 1) for e in ev) / args.steps
    for e in ev:
        e.close()
    _, st = lamp.lamp_decode_fwd(q, k, v, causal=w.causal, mu=args.mu, tau=tau, out=out,
                                 probs=probs, recompute_mask=mask, want_stats=True,
                                 ps_block=args.ps_block)
    n_valid = st["n_valid"]
    rate = st["n_selected"] / n_valid
    value = n_valid / (wall / args.steps)
    BH = B * H
    cache = BH * S * D * 4                       # K or V, read once
    chunks = (S + 255) // 256
    score_bytes = {
        # K; the queries; y^lo and y^ref written; block maxima
        "scores": cache + BH * nq * D * 4 + 8 * n_valid + 4 * BH * nq * ((S + 63) // 64),
        # V; y^lo and y^ref read; y^mix of the selected keys and the mask
        # written; the chunk partials
        "select": cache + 8 * n_valid + 4 * rate * n_valid + n_valid / 8
                  + BH * chunks * nq * (48 + 8 * D),
    }
    kstage = max(("scores", "select"), key=lambda n: stages[n])
    kname = {"scores": "decode_scores_kernel", "select": "decode_softmax_kernel"}[kstage]
    achieved = score_bytes[kstage] / (stages[kstage] * 1e-3)
    traffic = load_traffic(kname, f"{w.name}_nq{nq}")
    rec = {
        "metric": "LAMP decode scores/sec (relaxed, mu=4) + % HBM roofline", "value": value,
        "unit": "scores/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": 1e3 * wall / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "S": S, "D": D, "Nq": nq,
                   "causal": w.causal, "mu": args.mu, "mode": "relaxed",
                   "ps_block": args.ps_block, "tau": tau, "rate": rate,
                   "probs": probs is not None, "mask": True, "row_kl": True,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved / 1e9,
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": achieved / HBM_PEAK,
                     "traffic": traffic, "kernel_ms": stages[kstage],
                     "bytes_per_launch": score_bytes[kstage]},
        "path_alu_frac": (9 * D + 40) * value / ALU_PEAK,
        "stages_ms": stages,
        "kl_mean": st["kl_sum"] / st["n_rows"],
        "kl_lowp_mean": st["kl_lowp_sum"] / st["n_rows"],
        "exact_chunks": st["n_exact_tiles"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        rec["cpu_baseline"] = decode_cpu_baseline(Q, K, V, w, nq, args.mu, tau, args.ps_block)
    print(json.dumps(rec), flush=True)


def mlp_cpu_baseline(X, W, gamma, beta, w, mu, tau, ps_block=0):
    import numpy as np
    import oracle
    oracle.build(force=False)
    order = np.random.default_rng(0).permutation(w.M)
    threads = oracle.max_threads()
    done, dt = 0, 0.0
    while done < w.M and dt < CPU_TARGET_S:
        rows = np.sort(order[done:done + 64])
        t0 = time.perf_counter()
        ylo, yref = oracle.ps_gemm(X[rows], W, mu=mu, ps_block=ps_block)
        if w.op == "gelu":
            oracle.gelu_lamp(ylo, yref, tau=tau)
        else:
            oracle.ln_lamp(ylo, yref, gamma, beta, eps=w.eps, tau=tau)
        dt += time.perf_counter() - t0
        done += rows.size
    n = done * w.N
    return {"value": n / dt, "unit": "outputs/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.M} rows (all {w.N} columns, rows in a seeded random order) "
                      f"of {w.name}, same mu/tau; {n} outputs in {dt:.2f} s wall, "
                      f"{threads} OpenMP threads"}


def bench_mlp(args, w):
    """LAMP after a PS(mu) matrix product: y = x W^T, then GELU with the
    activation rule or layer normalisation with the greedy rule.  The
    dominant kernel is the fast-path product (the same 9-instruction PS(mu)
    multiply-add as the attention scores, plus the FP32 reference product),
    reported against the ALU peak with 9 K lane-operations per output."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    from mixed_precision_attention_ps_amd.configs import tau_for
    tau = args.tau if args.tau is not None else tau_for(w.name, w.op, args.mu, args.rate)
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name} {w.op} M={w.M} N={w.N} K={w.K} mu={args.mu} tau={tau}")
    X, W, gamma, beta = w.inputs()
    x, wt, g, b = (torch.from_numpy(a).to(dev) for a in (X, W, gamma, beta))
    M, N, K = w.M, w.N, w.K
    out = torch.empty((M, N), device=dev)
    mask = torch.empty((M, (N + 31) // 32), dtype=torch.int32, device=dev)
    row_err = torch.empty(M, dtype=torch.float64, device=dev)
    copy_calibration(args, dev)

    def step(events=None):
        if w.op == "gelu":
            lamp.lamp_gelu_fwd(x, wt, mu=args.mu, tau=tau, out=out, recompute_mask=mask,
                               row_err=row_err, want_stats=False, stage_events=events,
                               ps_block=args.ps_block)
        else:
            lamp.lamp_layernorm_fwd(x, wt, g, b, mu=args.mu, eps=w.eps, tau=tau, out=out,
                                    recompute_mask=mask, row_err=row_err, want_stats=False,
                                    stage_events=events, ps_block=args.ps_block)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [lamp.HipEvents(2 * lamp.LAMP_N_STAGES) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(ev[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = {}
    for name in ("scan", "exact", "scores", "finish"):
        si = lamp.STAGES.index(name)
        stages[name] = sum(e.elapsed_ms(2 * si, 2 * si + 1) for e in ev) / args.steps
    for e in ev:
        e.close()
    if w.op == "gelu":
        _, st = lamp.lamp_gelu_fwd(x, wt, mu=args.mu, tau=tau, out=out, want_stats=True,
                                   ps_block=args.ps_block)
    else:
        _, st = lamp.lamp_layernorm_fwd(x, wt, g, b, mu=args.mu, eps=w.eps, tau=tau, out=out,
                                        want_stats=True, ps_block=args.ps_block)
    n_out = M * N
    rate = st["n_selected"] / n_out
    value = n_out / (wall / args.steps)
    # the fast-path product kernel (64 x 64 or 32 x 32 tiles, whichever the
    # library picks for this shape; its traffic entry is keyed the same way)
    kname = "ps_gemm_kernel"
    w_alg = 9 * K + run_flush_ops(K, args.ps_block)
    t_kernel_ms = stages["scores"]
    achieved = w_alg * n_out / (t_kernel_ms * 1e-3)
    rec = {
        "metric": f"LAMP {w.op} outputs/sec after a PS(mu=4) matrix product + % VALU roofline",
        "value": value, "unit": "outputs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": 1e3 * wall / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "N": N, "K": K, "op": w.op, "mu": args.mu,
                   "ps_block": args.ps_block,
                   "tau": tau, "rate": rate, "mask": True, "row_err": True,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "alu", "kernel": kname, "achieved": achieved / 1e12,
                     "peak": ALU_PEAK / 1e12, "unit": "Tlane-op/s", "frac": achieved / ALU_PEAK,
                     "traffic": load_traffic(kname, w.name), "kernel_ms": t_kernel_ms,
                     "slots_per_output": w_alg},
        "path_alu_frac": w_alg * value / ALU_PEAK,
        "stages_ms": stages,
        "err_mean": st["kl_sum"] / st["n_rows"],
        "err_lowp_mean": st["kl_lowp_sum"] / st["n_rows"],
        "exact_tiles": st["n_exact_tiles"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        rec["cpu_baseline"] = mlp_cpu_baseline(X, W, gamma, beta, w, args.mu, tau,
                                               args.ps_block)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_xl_layer")
    ap.add_argument("--mode", default="strict", choices=["strict", "relaxed", "random"])
    ap.add_argument("--mu", type=int, default=4)
    ap.add_argument("--rate", type=float, default=0.016, help="target recompute rate (tau table)")
    ap.add_argument("--tau", type=float, default=None, help="explicit tau (overrides --rate)")
    ap.add_argument("--no-probs", action="store_true")
    ap.add_argument("--no-kl", action="store_true",
                    help="attention: no row KL in the timed calls (the serving case)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-relaxed", action="store_true",
                    help="strict runs: no relaxed sub-record (the library's choice and the "
                         "fused kernel on the same layer)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    ap.add_argument("--nq", type=int, default=1, help="decode workloads: queries per head")
    ap.add_argument("--relaxed-path", type=int, default=0, choices=[0, 1, 2],
                    help="relaxed mode: 0 the library's choice, 1 the fused one-pass kernel, "
                         "2 score tiles then the row pass (rows of <= 1024 keys)")
    ap.add_argument("--ps-block", type=int, default=0,
                    help="PS(mu) accumulation order: 0 sequential, else runs of this many "
                         "products (blocked order)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: every LAMP quantity is per query row, so a layer "
              "shards over (batch, head) with no exchange and each GPU would run this same "
              "benchmark on its share; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixed_precision_attention_ps_amd import lamp
    from mixed_precision_attention_ps_amd.configs import MLP_WORKLOADS, WORKLOADS

    if args.workload in MLP_WORKLOADS:
        return bench_mlp(args, MLP_WORKLOADS[args.workload])
    w = WORKLOADS[args.workload]
    if w.name.startswith("decode"):
        return bench_decode(args, w)
    dev = torch.device("cuda:0")
    Q, K, V, _ = w.qkv()
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    copy_calibration(args, dev)

    rec = measure_attention(args, w, lamp, torch, q, k, v, args.mode, args.relaxed_path,
                            args.steps, args.warmup)
    if args.mode == "strict" and not args.no_relaxed:
        # the relaxed rule on the same layer and inputs: the implementation
        # the library picks, and the fused one-pass kernel
        sub = {}
        for name, rp in (("library_choice", 0), ("fused_kernel", 1)):
            r = measure_attention(args, w, lamp, torch, q, k, v, "relaxed", rp, args.steps,
                                  args.warmup)
            sub[name] = {key: r[key] for key in ("value", "ms_per_step", "gpu_ms_per_step",
                                                 "roofline", "path_alu_frac", "stages_ms",
                                                 "kl_mean", "kl_reduction")}
            sub[name]["impl"] = r["config"]["impl"]
            sub[name]["tau"] = r["config"]["tau"]
            sub[name]["rate"] = r["config"]["rate"]
            sub[name]["relaxed_path"] = rp
        rec["relaxed"] = sub
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        mode_id = lamp.MODES[args.mode]
        rec["cpu_baseline"] = cpu_baseline(Q, K, V, w, mode_id, args.mu, rec["config"]["tau"], 0,
                                           args.ps_block)
    print(json.dumps(rec), flush=True)


def measure_attention(args, w, lamp, torch, q, k, v, mode, relaxed_path, steps, warmup):
    """Times `steps` lamp_attention_fwd calls (after `warmup`) in one mode on
    the resident inputs; returns the record of that measurement."""
    mode_id = lamp.MODES[mode]
    tau_mode = "strict" if mode == "random" else mode
    tau = args.tau if args.tau is not None else tau_for_workload(w.name, tau_mode, args.mu,
                                                                 args.rate)
    dev = q.device
    log(f"[bench] {w.name} mode={mode} mu={args.mu} tau={tau} relaxed_path={relaxed_path}")
    B, H, S, D = w.B, w.H, w.S, w.D
    W32 = (S + 31) // 32
    out = torch.empty_like(q)
    probs = None if args.no_probs else torch.empty((B, H, S, S), device=dev)
    mask = torch.empty((B, H, S, W32), dtype=torch.int32, device=dev)
    row_kl = torch.empty((B, H, S), dtype=torch.float64, device=dev)

    def step(events=None):
        lamp.lamp_attention_fwd(q, k, v, causal=w.causal, mu=args.mu, tau=tau, mode=mode_id,
                                out=out, probs=probs, recompute_mask=mask, want_stats=False,
                                row_kl=None if args.no_kl else row_kl, stage_events=events,
                                ps_block=args.ps_block, relaxed_path=relaxed_path)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timing-only events (no cache write-back on record) around every stage
    # of the timed steps
    ev = [lamp.HipEvents(2 * lamp.LAMP_N_STAGES) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for s in range(steps):
        step(ev[s])
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = t_start.elapsed_time(t_stop)

    # the implementation the library ran (it reports it; the stage events
    # that implementation records are the ones read)
    impl = lamp.last_impl()
    if impl == "relaxed_fused":
        ran = ["scan", "exact", "scores"] + (["finish"] if probs is not None else [])
    elif impl in ("strict_rows", "relaxed_rows"):
        # the fused row pass and P.V (with the row KLs)
        ran = ["scan", "exact", "scores", "select"]
    elif impl == "relaxed_stream":
        # the streaming relaxed row pass of longer rows, then P.V
        ran = ["scan", "exact", "scores", "select", "finish"]
    else:
        ran = ["scan", "exact", "scores", "select", "recompute", "finish"]
    stages = {}
    for name in ran:
        si = lamp.STAGES.index(name)
        stages[name] = sum(e.elapsed_ms(2 * si, 2 * si + 1) for e in ev) / steps
    for e in ev:
        e.close()

    # untimed: rate and KL of the same call
    _, st = lamp.lamp_attention_fwd(q, k, v, causal=w.causal, mu=args.mu, tau=tau, mode=mode_id,
                                    out=out, probs=probs, recompute_mask=mask, want_stats=True,
                                    ps_block=args.ps_block, relaxed_path=relaxed_path)
    del out, probs, mask, row_kl
    n_valid = st["n_valid"]
    rate = st["n_selected"] / n_valid
    ms_per_step = 1e3 * wall / steps
    value = n_valid / (wall / steps)

    # dominant kernel: the PS(mu)+FP32 score tiles (strict, random, relaxed in
    # two passes) or the fused relaxed kernel; algorithmic VALU slots per valid
    # score: 8D (PS(mu) dot: multiply, add, two 3-instruction roundings per
    # MAC) + D (FP32 reference dot at two lanes per slot) [+ 20 for the fused
    # softmax/criterion/KL].
    fused_relaxed = impl == "relaxed_fused"
    kname = "relaxed_kernel" if fused_relaxed else "ps_scores_kernel"
    w_alg = 9 * D + (20 if fused_relaxed else 0) + run_flush_ops(D, args.ps_block)
    t_kernel_ms = stages.get("scores")
    achieved = w_alg * n_valid / (t_kernel_ms * 1e-3) if t_kernel_ms else None
    traffic = load_traffic(kname, w.name)
    roofline = {"bound": "alu", "kernel": kname,
                "achieved": achieved / 1e12 if achieved else None,
                "peak": ALU_PEAK / 1e12, "unit": "Tlane-op/s",
                "frac": achieved / ALU_PEAK if achieved else None,
                "traffic": traffic, "kernel_ms": t_kernel_ms,
                "slots_per_score": w_alg}
    # whole path against the same peak (8D + D + 20 + 2 r D per score) and HBM
    w_path = 9 * D + 20 + 2 * rate * D + run_flush_ops(D, args.ps_block)
    # the same work against the single-pipe 16-lane VALU rate (256 CUs x 4 SIMDs
    # x 16 lanes x 2.4 GHz = 3.93e13 lane-slots/s), counting the FP32 reference
    # dot at two lanes per slot as above: the convention of a pure 16-lane
    # machine, which the measured co-issue of FP32 and integer work exceeds
    VALU16_PEAK = 256 * 4 * 16 * 2.4e9
    hbm_bytes = (0 if args.no_probs else 4) + 1 / 8 + 32 * D / (S + 1)
    return {
        "metric": METRIC, "value": value, "unit": "scores/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "S": S, "D": D, "causal": w.causal,
                   "mu": args.mu, "mode": mode, "ps_block": args.ps_block, "tau": tau,
                   "impl": impl,
                   "target_rate": args.rate,
                   "rate": rate, "probs": not args.no_probs, "mask": True,
                   "row_kl": not args.no_kl,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "path_alu_frac": w_path * value / ALU_PEAK,
        "path_valu16_frac": w_path * value / VALU16_PEAK,
        "path_hbm_frac": hbm_bytes * value / HBM_PEAK,
        "gpu_ms_per_step": gpu_ms / steps,
        "stages_ms": stages,
        "kl_mean": st["kl_sum"] / st["n_rows"],
        "kl_lowp_mean": st["kl_lowp_sum"] / st["n_rows"],
        "kl_reduction": (st["kl_lowp_sum"] / st["kl_sum"]) if st["kl_sum"] > 0 else None,
        "exact_tiles": st["n_exact_tiles"],
    }


if __name__ == "__main__":
    main()

"""Find thresholds tau that hit target recompute rates, on the CPU oracle.

Writes mixed_precision_attention_ps_amd/tau_table.json.  Only the oracle and
the seeded input generator are used.  For each workload and mode the oracle's
criterion values (strict: 2 z (1 - z) |y^lo|; relaxed: 2 exp(y^lo - m_t)
|y^lo|) are collected over a sample of heads (and rows), and tau is the FP32
value at which the fraction of valid scores whose criterion exceeds tau is the
target rate.  After a matrix product the GELU criterion |GELU'(y) y| is
collected the same way; the layer-normalisation rule has no per-element
criterion, so its tau is found by bisection on the oracle's row counts.  The
thresholds are inputs of the benchmark; the rate a run actually reaches is
measured by that run.

Usage: python oracle/calibrate_tau.py [workload ...]   (default: all; named
workloads are recalibrated and merged into the existing table)
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mixed_precision_attention_ps_amd.configs import MLP_WORKLOADS, WORKLOADS  # noqa: E402

OUT = os.path.join(ROOT, "mixed_precision_attention_ps_amd", "tau_table.json")
RATES = (0.003, 0.016, 0.076)


def tau_for_rate(crit: np.ndarray, rate: float) -> float:
    c = np.sort(crit)[::-1]
    k = int(round(rate * c.size))
    k = min(max(k, 1), c.size - 1)
    tau = np.float32(0.5 * (c[k - 1] + c[k]))   # between the k-th and (k+1)-th largest
    return float(tau)


def collect(w, mode, mu, heads, row_ranges):
    Q, K, V, _ = w.qkv()
    parts = []
    for rows in row_ranges:
        r = oracle.lamp_heads(Q, K, V, causal=w.causal, mu=mu, tau=np.inf, mode=mode, heads=heads,
                              rows=rows, want=("crit",))
        S = w.S
        rb, re_ = rows
        i = np.arange(rb, re_)[:, None]
        valid = (np.arange(S)[None, :] <= i) if w.causal else np.ones((re_ - rb, S), bool)
        parts.append(r["crit"][:, valid])
    return np.concatenate([p.ravel() for p in parts])


MLP_SAMPLE_ROWS = list(range(0, 1024, 32))


def calibrate_mlp(table, name):
    w = MLP_WORKLOADS[name]
    for mu in w.mus:
        calibrate_mlp_mu(table, w, mu)


def calibrate_mlp_mu(table, w, mu):
    X, W, gamma, beta = w.inputs()
    ylo, yref = oracle.ps_gemm(X[MLP_SAMPLE_ROWS], W, mu=mu)
    sample = f"rows {MLP_SAMPLE_ROWS[0]}..{MLP_SAMPLE_ROWS[-1]} step 32, all columns"
    rate = 0.016
    if w.op == "gelu":
        crit = oracle.gelu_lamp(ylo, yref, tau=np.inf)["crit"].ravel()
        tau = tau_for_rate(crit, rate)
        got = float((crit > np.float32(tau)).mean())
    else:
        # the rate falls as tau grows: bisect over float32 values of tau
        def frac(t):
            return oracle.ln_lamp(ylo, yref, gamma, beta, eps=w.eps, tau=t)["count"].sum() / ylo.size
        lo, hi = 0.0, 4.0
        for _ in range(60):
            mid = float(np.float32(0.5 * (lo + hi)))
            if mid in (lo, hi):
                break
            if frac(mid) > rate:
                lo = mid
            else:
                hi = mid
        tau = hi
        got = float(frac(tau))
    table[f"{w.name}/{w.op}/mu{mu}/rate{rate}"] = {"tau": tau, "sample_rate": got, "sample": sample}
    print(w.name, w.op, mu, tau, got, flush=True)


def main():
    names = sys.argv[1:]
    if names:
        with open(OUT) as f:
            table = json.load(f)
        for n in names:
            if n not in MLP_WORKLOADS:
                raise SystemExit(f"only the matrix-product workloads can be recalibrated alone: {n}")
            calibrate_mlp(table, n)
        with open(OUT, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)
        print("wrote", OUT)
        return
    table = {}
    for n in MLP_WORKLOADS:
        calibrate_mlp(table, n)
    w = WORKLOADS["gpt2_xl_layer"]
    heads = [0, 33, 66, 99, 133, 166, 199]
    for mode_name, mode in (("strict", oracle.STRICT), ("relaxed", oracle.RELAXED)):
        for mu in w.mus:
            crit = collect(w, mode, mu, heads, [(0, w.S)])
            for rate in RATES:
                tau = tau_for_rate(crit, rate)
                table[f"{w.name}/{mode_name}/mu{mu}/rate{rate}"] = {
                    "tau": tau, "sample_rate": float((crit > np.float32(tau)).mean()),
                    "sample": f"heads {heads}, all rows"}
                print(w.name, mode_name, mu, rate, tau, flush=True)
    w = WORKLOADS["long_context_s16384"]
    rows = [(0, 64), (4096, 4160), (8192, 8256), (12288, 12352), (16320, 16384)]
    for mode_name, mode in (("relaxed", oracle.RELAXED), ("strict", oracle.STRICT)):
        crit = collect(w, mode, 4, [0, 31], rows)
        tau = tau_for_rate(crit, 0.016)
        table[f"{w.name}/{mode_name}/mu4/rate0.016"] = {
            "tau": tau, "sample_rate": float((crit > np.float32(tau)).mean()),
            "sample": f"heads [0, 31], rows {rows}"}
        print(w.name, mode_name, tau, flush=True)
    w = WORKLOADS["decode_s16384"]
    rows = [(w.S - 16, w.S)]
    crit = collect(w, oracle.RELAXED, 4, [0, 50, 99, 150, 199], rows)
    tau = tau_for_rate(crit, 0.016)
    table[f"{w.name}/relaxed/mu4/rate0.016"] = {
        "tau": tau, "sample_rate": float((crit > np.float32(tau)).mean()),
        "sample": f"heads [0, 50, 99, 150, 199], rows {rows} (the decode queries)"}
    print(w.name, "relaxed", tau, flush=True)
    with open(OUT, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print("wrote", OUT)


if __name__ == "__main__":
    main()

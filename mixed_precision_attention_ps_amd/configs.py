"""The synthetic LAMP workloads and their thresholds.

Shapes, distributions and (mu, mode, tau) sweeps of the workloads the build is
measured and checked on.  The GPT-2 shapes mirror the models the LAMP
summary's "Experimental results" section evaluates (GPT-2 XL: 25 heads of
width 64); the activations themselves are synthetic (see ``inputs``).

``TAU_FOR_RATE`` holds thresholds that hit target recompute rates on the
GPT-2-XL-shaped layer.  They were found by bisection on the CPU oracle over a
sample of heads (``oracle/calibrate_tau.py`` writes them); they are inputs, not
expected values.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    n_outlier: int = 0
    outlier_factor: float = 8.0
    qk_std: float = 1.0
    mus: tuple = (4,)
    mode: str = "strict"
    taus: tuple = ()
    seed: int = 0

    @property
    def n_valid(self) -> int:
        per_head = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return self.B * self.H * per_head

    def qkv(self, seed=None):
        from .inputs import make_qkv
        return make_qkv(self.B, self.H, self.S, self.D, n_outlier=self.n_outlier,
                        outlier_factor=self.outlier_factor, qk_std=self.qk_std,
                        seed=self.seed if seed is None else seed)


WORKLOADS = {
    w.name: w for w in [
        Workload("single_head_s128", 1, 1, 128, 64, False, 0, 1.0, 1.0, (4,), "strict",
                 (1e-1, 1e-2, 1e-3)),
        Workload("gpt2_small_s1024", 1, 12, 1024, 64, True, 2, 8.0, 1.0, (4,), "strict",
                 (1e-1, 1e-2, 1e-3, 1e-4)),
        Workload("gpt2_xl_layer", 8, 25, 1024, 64, True, 2, 8.0, 1.0, (4, 7, 10), "strict"),
        Workload("relaxed_s4096", 4, 25, 4096, 64, True, 4, 8.0, 1.0, (4,), "relaxed",
                 (1e-1, 1e-2, 1e-3, 1e-4)),
        Workload("long_context_s16384", 1, 32, 16384, 128, True, 1, 16.0, 0.5, (4,), "relaxed"),
        # decode shapes: the last Nq rows of Q (Nq <= 16) against a 16K-key
        # cache, GPT-2-XL heads (8 x 25, D = 64, 2 outlier channels x8)
        Workload("decode_s16384", 8, 25, 16384, 64, True, 2, 8.0, 1.0, (4,), "relaxed"),
    ]
}

@dataclass(frozen=True)
class MlpWorkload:
    """y = X W^T (X [M, K], W [N, K]) followed by GELU or layer normalisation."""
    name: str
    M: int
    N: int
    K: int
    op: str              # "gelu" or "layernorm"
    w_std: float = 0.02
    eps: float = 1e-5
    mus: tuple = (4,)
    seed: int = 0

    @property
    def n_valid(self) -> int:
        return self.M * self.N

    def inputs(self, seed=None):
        from .inputs import make_mlp
        return make_mlp(self.M, self.N, self.K, w_std=self.w_std,
                        seed=self.seed if seed is None else seed)


MLP_WORKLOADS = {
    w.name: w for w in [
        # GPT-2 XL MLP up-projection of 1024 tokens (d_model 1600 -> 6400)
        # followed by the activation
        MlpWorkload("gelu_gpt2_xl_mlp", 1024, 6400, 1600, "gelu", mus=(4, 7, 10)),
        # GPT-2 XL MLP down-projection (6400 -> 1600) followed by a layer norm
        MlpWorkload("ln_gpt2_xl", 1024, 1600, 6400, "layernorm", mus=(4, 7, 10)),
    ]
}


def _load_tau_table() -> dict:
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tau_table.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)


# Written by oracle/calibrate_tau.py: "workload/mode/mu<m>/rate<r>" -> {"tau": ...}.
TAU_TABLE: dict = _load_tau_table()


def tau_for(workload: str, mode: str, mu: int, rate: float) -> float:
    key = f"{workload}/{mode}/mu{mu}/rate{rate}"
    if key not in TAU_TABLE:
        raise KeyError(f"no calibrated tau for {key}; run oracle/calibrate_tau.py")
    return float(TAU_TABLE[key]["tau"])

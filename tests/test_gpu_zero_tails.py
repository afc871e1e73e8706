"""GPU tests of the causal probabilities' zero tails.

Under a causal mask the probabilities of row i are 0 at every key past i.
The zeros past a row's own 64-key block are written by the kernel that runs
beside the ALU-bound score work (the score tiles, each zero-filling its
mirrored upper tile, or the fused relaxed kernel, each query block its own
rows), and the row passes write only up to the end of the block.  Each
implementation is run here on a probabilities buffer filled with NaN, at
lengths that are not multiples of 64 (and one that is not a multiple of 4,
where the stores are 4-byte ones), with y^lo kept in place in the
probabilities buffer (no scores asked for): every entry above the diagonal
must be exactly +0, and the rest must match the oracle (tests/parity.py
bars).  The strict rule also runs at mu = 12 and 23 (every tile on the
generic kernel, which then writes the zero tiles) and in a blocked order
(diagonal tiles in the plain tile loop).
"""
import sys

import numpy as np
import pytest

from mixed_precision_attention_ps_amd.inputs import make_qkv
from tests import parity
from tests.test_gpu_parity import RANDOM, RELAXED, STRICT, compare_full, run_orc

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


_ORC = {}


def oracle_for(orc, Q, K, V, S, mode, tau, mu=4, ps_block=0):
    key = (S, mode, mu, ps_block)
    if key not in _ORC:
        _ORC[key] = run_orc(orc, Q, K, V, causal=True, mu=mu, tau=tau, mode=mode, seed=5,
                            ps_block=ps_block)
    return _ORC[key]


@pytest.mark.parametrize("S", [202, 1090, 1156])
@pytest.mark.parametrize("mode,path,impls", [
    (STRICT, 0, ("strict_rows", "strict_stream")),
    (RELAXED, 0, ("relaxed_rows", "relaxed_stream")),
    (RELAXED, 1, ("relaxed_fused",)),
    (RANDOM, 0, ("random",)),
])
def test_causal_zero_tails_on_a_nan_buffer(dev, orc, S, mode, path, impls):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, D = 1, 2, 64
    tau = 1e-2
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=40 + S)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    W = (S + 31) // 32
    probs = torch.full((B, H, S, S), float("nan"), device=dev)
    mask = torch.full((B, H, S, W), -1, dtype=torch.int32, device=dev)
    note(f"zero tails mode={mode} relaxed_path={path} S={S}")
    out, st = lamp.lamp_attention_fwd(q, k, v, causal=True, mu=4, tau=tau, mode=mode,
                                      probs=probs, recompute_mask=mask, seed=5,
                                      want_stats=True, relaxed_path=path)
    torch.cuda.synchronize()
    assert lamp.IMPLS[st["impl"]] in impls
    p = probs.cpu().numpy().reshape(B * H, S, S)
    upper = ~parity.valid_mask(S, True)
    tail = p[:, upper]
    assert (tail == 0.0).all() and not np.signbit(tail).any(), "nonzero above the diagonal"
    g = {"out": out.cpu().numpy(), "probs": probs.cpu().numpy(),
         "mask": mask.cpu().numpy().view(np.uint32), "stats": st}
    r = oracle_for(orc, Q, K, V, S, mode, tau)
    if mode == RANDOM:
        assert (g["mask"].reshape(-1, S, W) == r["mask"]).all()
    compare_full(g, r, Q, V, causal=True, tau=np.inf if mode == RANDOM else tau)


@pytest.mark.parametrize("mu,ps_block", [(12, 0), (23, 0), (4, 16)])
def test_zero_tails_generic_and_blocked_paths(dev, orc, mu, ps_block):
    """mu > 10 (every tile on the generic kernel, which then writes the zero
    tiles) and a blocked order (diagonal tiles in the plain tile loop)."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    B, H, S, D = 1, 2, 202, 64
    tau = 1e-2
    Q, K, V, _ = make_qkv(B, H, S, D, n_outlier=2, seed=70 + mu)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    W = (S + 31) // 32
    probs = torch.full((B, H, S, S), float("nan"), device=dev)
    mask = torch.full((B, H, S, W), -1, dtype=torch.int32, device=dev)
    note(f"zero tails strict mu={mu} ps_block={ps_block} S={S}")
    out, st = lamp.lamp_attention_fwd(q, k, v, causal=True, mu=mu, tau=tau, mode=STRICT,
                                      probs=probs, recompute_mask=mask, want_stats=True,
                                      ps_block=ps_block)
    torch.cuda.synchronize()
    p = probs.cpu().numpy().reshape(B * H, S, S)
    tail = p[:, ~parity.valid_mask(S, True)]
    assert (tail == 0.0).all() and not np.signbit(tail).any(), "nonzero above the diagonal"
    g = {"out": out.cpu().numpy(), "probs": probs.cpu().numpy(),
         "mask": mask.cpu().numpy().view(np.uint32), "stats": st}
    r = oracle_for(orc, Q, K, V, S, STRICT, tau, mu=mu, ps_block=ps_block)
    compare_full(g, r, Q, V, causal=True, tau=tau)

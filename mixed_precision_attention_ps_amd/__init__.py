"""LAMP attention forward on MI355X (gfx950).

Look-Ahead Mixed-Precision attention: K.Q scores with emulated PS(mu)
accumulation, closed-form look-ahead selection (strict, relaxed, random
control), FP32 recompute of the selected scores, softmax, P.V and a row-wise
KL(FP32 || LAMP), all in hand-written HIP kernels behind the C ABI declared in
``include/lamp.h``.

Importing this package loads nothing: ``inputs`` and ``configs`` are plain
numpy; the HIP library is loaded by ``mixed_precision_attention_ps_amd.lamp``.
"""
__all__ = ["inputs", "configs", "lamp"]

"""Python binding of the LAMP C ABI (include/lamp.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``liblamp.so``.  Tensors are torch CUDA (ROCm) float32 tensors,
used for their device pointers; work is enqueued on torch's current stream.
The library must be built (``__graft_entry__.build()``); loading fails loudly
otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LAMP_STRICT, LAMP_RELAXED, LAMP_RANDOM = 0, 1, 2
MODES = {"strict": LAMP_STRICT, "relaxed": LAMP_RELAXED, "random": LAMP_RANDOM}
LAMP_OK, LAMP_ERR_INVALID_ARG, LAMP_ERR_UNSUPPORTED, LAMP_ERR_HIP, LAMP_ERR_NO_MEMORY = 0, -1, -2, -3, -4
STAGES = ("scan", "scores", "select", "recompute", "finish", "stats", "exact")
LAMP_N_STAGES = len(STAGES)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblamp.so")


IMPLS = {0: "none", 1: "strict_rows", 2: "strict_stream", 3: "random", 4: "relaxed_fused",
         5: "relaxed_rows", 6: "relaxed_stream", 7: "decode", 8: "gelu", 9: "layernorm"}


class LampStats(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_uint64), ("n_valid", ctypes.c_uint64),
                ("n_selected", ctypes.c_uint64), ("n_exact_tiles", ctypes.c_uint64),
                ("kl_sum", ctypes.c_double), ("kl_max", ctypes.c_double),
                ("kl_lowp_sum", ctypes.c_double), ("n_tie_band", ctypes.c_uint64),
                ("impl", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class LampParams(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("seed", ctypes.c_uint64),
                ("row_kl", ctypes.c_void_p), ("row_kl_lowp", ctypes.c_void_p),
                ("row_count", ctypes.c_void_p), ("scores_mix", ctypes.c_void_p),
                ("scores_ref", ctypes.c_void_p), ("stage_events", ctypes.c_void_p),
                ("ps_block", ctypes.c_int), ("relaxed_path", ctypes.c_int),
                ("block_k", ctypes.c_int)]


class LampError(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        super().__init__(f"LAMP error {code}: {detail}")


_lib = None


def library():
    """Load liblamp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd_args = [P, P, P, I, I, I, I, I, I, F, I, P, P, P, ctypes.POINTER(LampStats)]
    lib.lamp_attention_fwd.restype = I
    lib.lamp_attention_fwd.argtypes = fwd_args
    lib.lamp_attention_fwd_ex.restype = I
    lib.lamp_attention_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(LampParams)]
    lib.lamp_attention_fwd_noalloc.restype = I
    lib.lamp_attention_fwd_noalloc.argtypes = fwd_args + [ctypes.POINTER(LampParams)]
    lib.lamp_workspace_bytes.restype = ctypes.c_size_t
    lib.lamp_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.lamp_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.lamp_workspace_bytes_ex.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(LampParams)]
    lib.lamp_ps_scores.restype = I
    lib.lamp_ps_scores.argtypes = [P, P, I, I, I, I, I, I, P, P, P]
    lib.lamp_strerror.restype = ctypes.c_char_p
    lib.lamp_strerror.argtypes = [I]
    lib.lamp_last_error.restype = ctypes.c_char_p
    lib.lamp_last_error.argtypes = []
    lib.lamp_version.restype = I
    lib.lamp_version.argtypes = []
    lib.lamp_last_impl.restype = I
    lib.lamp_last_impl.argtypes = []
    lib.lamp_diag_exp.restype = I
    lib.lamp_diag_exp.argtypes = [P, P, P, I, P]
    lib.lamp_decode_fwd.restype = I
    lib.lamp_decode_fwd.argtypes = [P, P, P, I, I, I, I, I, I, I, F, P, P, P,
                                    ctypes.POINTER(LampStats), ctypes.POINTER(LampParams)]
    lib.lamp_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.lamp_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.lamp_gelu_fwd.restype = I
    lib.lamp_gelu_fwd.argtypes = [P, P, I, I, I, I, F, P, P, ctypes.POINTER(LampStats),
                                  ctypes.POINTER(LampParams)]
    lib.lamp_layernorm_fwd.restype = I
    lib.lamp_layernorm_fwd.argtypes = [P, P, P, P, I, I, I, I, F, F, P, P,
                                       ctypes.POINTER(LampStats), ctypes.POINTER(LampParams)]
    lib.lamp_mlp_workspace_bytes.restype = ctypes.c_size_t
    lib.lamp_mlp_workspace_bytes.argtypes = [I, I, I, I]
    lib.lamp_gemm_scores.restype = I
    lib.lamp_gemm_scores.argtypes = [P, P, I, I, I, I, P, P, P]
    _lib = lib
    return lib


def _rc(rc: int):
    if rc != LAMP_OK:
        lib = library()
        detail = (lib.lamp_last_error() or b"").decode() or lib.lamp_strerror(rc).decode()
        raise LampError(rc, detail)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t, name):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


_INT32 = (torch.int32, torch.uint32)


def _check(t, name, shape, dtypes, device):
    """A tensor the library will read or write: a contiguous tensor of exactly
    `shape`, one of `dtypes`, on `device` (a wrong size would let the kernels
    run past its allocation).  None passes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def _check_workspace(ws, device):
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")


def last_impl() -> str:
    """Name of the implementation the calling thread's last successful call ran."""
    return IMPLS.get(int(library().lamp_last_impl()), "unknown")


def lamp_diag_exp(x):
    """The library's double and FP32-accurate exponentials of a float64 tensor."""
    y64 = torch.empty_like(x)
    y32 = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    rc = library().lamp_diag_exp(_ptr(x), _ptr(y64), _ptr(y32), x.numel(), stream)
    if rc != 0:
        raise LampError(rc, "lamp_diag_exp failed")
    return y64, y32


def lamp_workspace_bytes(B, H, S, D, mode, want_probs) -> int:
    return int(library().lamp_workspace_bytes(B, H, S, D, MODES.get(mode, mode), int(want_probs)))


def lamp_workspace_bytes_ex(B, H, S, D, causal, mode, want_probs, want_stats,
                            params: "LampParams | None" = None) -> int:
    """Exact workspace of one lamp_attention_fwd_ex call with these params."""
    p = ctypes.byref(params) if params is not None else None
    return int(library().lamp_workspace_bytes_ex(B, H, S, D, int(causal), MODES.get(mode, mode),
                                                 int(want_probs), int(want_stats), p))


def lamp_ps_scores(q, k, *, causal: bool, mu: int, ylo=None, yref=None):
    """Step 1 alone: PS(mu) scores and FP32 scores into [B,H,S,S] buffers."""
    B, H, S, D = q.shape
    _check(k, "k", (B, H, S, D), (torch.float32,), q.device)
    if ylo is None and yref is None:
        ylo = torch.empty((B, H, S, S), device=q.device, dtype=torch.float32)
        yref = torch.empty_like(ylo)
    for name, t in (("ylo", ylo), ("yref", yref)):
        _check(t, name, (B, H, S, S), (torch.float32,), q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    _rc(library().lamp_ps_scores(_f32(q, "q"), _f32(k, "k"), B, H, S, D, int(causal), int(mu),
                                    _ptr(ylo), _ptr(yref), stream))
    return ylo, yref


def lamp_attention_fwd(q, k, v, *, causal: bool, mu: int, tau: float, mode="strict", out=None,
                       probs=None, recompute_mask=None, want_stats: bool = True, seed: int = 0,
                       row_kl=None, row_kl_lowp=None, row_count=None, scores_mix=None,
                       scores_ref=None, workspace=None, stage_events=None, ps_block: int = 0,
                       relaxed_path: int = 0, block_k: int = 0, noalloc: bool = False):
    """LAMP attention forward through lamp_attention_fwd_ex (or, with
    noalloc=True, lamp_attention_fwd_noalloc: no workspace, the library's
    fixed scratch array).

    q, k, v: float32 [B, H, S, D] device tensors.  Optional outputs are written
    in place when given.  relaxed_path (relaxed mode): 0 the library's choice,
    1 the fused one-pass kernel, 2 two passes (score tiles, then a row pass).
    Returns (out, stats_dict_or_None).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, S, D = q.shape
    dev = q.device
    W = (S + 31) // 32
    if out is None:
        out = torch.empty_like(q)
    f32, f64 = (torch.float32,), (torch.float64,)
    for name, t, shape, dt in (
            ("k", k, (B, H, S, D), f32), ("v", v, (B, H, S, D), f32),
            ("out", out, (B, H, S, D), f32), ("probs", probs, (B, H, S, S), f32),
            ("recompute_mask", recompute_mask, (B, H, S, W), _INT32),
            ("row_kl", row_kl, (B, H, S), f64), ("row_kl_lowp", row_kl_lowp, (B, H, S), f64),
            ("row_count", row_count, (B, H, S), _INT32),
            ("scores_mix", scores_mix, (B, H, S, S), f32),
            ("scores_ref", scores_ref, (B, H, S, S), f32)):
        _check(t, name, shape, dt, dev)
    _check_workspace(workspace, dev)
    m = MODES.get(mode, mode)
    p = LampParams()
    p.stream = torch.cuda.current_stream(q.device).cuda_stream
    p.seed = seed & 0xFFFFFFFFFFFFFFFF
    p.ps_block = int(ps_block)
    p.relaxed_path = int(relaxed_path)
    p.block_k = int(block_k)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    for name, t in (("row_kl", row_kl), ("row_kl_lowp", row_kl_lowp), ("row_count", row_count),
                    ("scores_mix", scores_mix), ("scores_ref", scores_ref)):
        if t is not None:
            setattr(p, name, _ptr(t).value)
    if stage_events is not None:   # a HipEvents of 2 * LAMP_N_STAGES handles
        p.stage_events = stage_events.address
    st = LampStats() if want_stats else None
    mask_ptr = None
    if recompute_mask is not None:
        if recompute_mask.dtype not in (torch.int32, torch.uint32):
            raise TypeError("recompute_mask must be a 32-bit integer tensor")
        mask_ptr = _ptr(recompute_mask)
    if noalloc and workspace is not None:
        raise ValueError("the allocation-free entry point takes no workspace")
    fn = library().lamp_attention_fwd_noalloc if noalloc else library().lamp_attention_fwd_ex
    _rc(fn(
        _f32(q, "q"), _f32(k, "k"), _f32(v, "v"), B, H, S, D, int(causal), int(mu),
        ctypes.c_float(tau), int(m), _f32(out, "out"),
        None if probs is None else _f32(probs, "probs"), mask_ptr,
        ctypes.byref(st) if st is not None else None, ctypes.byref(p)))
    return out, (st.as_dict() if st is not None else None)


def lamp_decode_fwd(q, k, v, *, causal: bool, mu: int, tau: float, out=None, probs=None,
                    recompute_mask=None, want_stats: bool = True, row_kl=None, row_kl_lowp=None,
                    row_count=None, scores_mix=None, scores_ref=None, workspace=None,
                    stage_events=None, ps_block: int = 0):
    """Relaxed LAMP at decode shapes through lamp_decode_fwd.

    q: float32 [B, H, Nq, D]; k, v: float32 [B, H, S, D] device tensors (the
    queries are the last Nq positions of the sequence).  Optional outputs are
    written in place when given.  Returns (out, stats_dict_or_None).
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, D] and k [B, H, S, D]")
    B, H, Nq, D = q.shape
    S = k.shape[2]
    if tuple(k.shape) != (B, H, S, D) or tuple(v.shape) != (B, H, S, D):
        raise ValueError("k and v must be [B, H, S, D] with q's B, H, D")
    dev = q.device
    W = (S + 31) // 32
    if out is None:
        out = torch.empty_like(q)
    f32, f64 = (torch.float32,), (torch.float64,)
    for name, t, shape, dt in (
            ("k", k, (B, H, S, D), f32), ("v", v, (B, H, S, D), f32),
            ("out", out, (B, H, Nq, D), f32), ("probs", probs, (B, H, Nq, S), f32),
            ("recompute_mask", recompute_mask, (B, H, Nq, W), _INT32),
            ("row_kl", row_kl, (B, H, Nq), f64), ("row_kl_lowp", row_kl_lowp, (B, H, Nq), f64),
            ("row_count", row_count, (B, H, Nq), _INT32),
            ("scores_mix", scores_mix, (B, H, Nq, S), f32),
            ("scores_ref", scores_ref, (B, H, Nq, S), f32)):
        _check(t, name, shape, dt, dev)
    _check_workspace(workspace, dev)
    p = LampParams()
    p.stream = torch.cuda.current_stream(q.device).cuda_stream
    p.ps_block = int(ps_block)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    for name, t in (("row_kl", row_kl), ("row_kl_lowp", row_kl_lowp), ("row_count", row_count),
                    ("scores_mix", scores_mix), ("scores_ref", scores_ref)):
        if t is not None:
            setattr(p, name, _ptr(t).value)
    if stage_events is not None:
        p.stage_events = stage_events.address
    st = LampStats() if want_stats else None
    mask_ptr = None
    if recompute_mask is not None:
        if recompute_mask.dtype not in (torch.int32, torch.uint32):
            raise TypeError("recompute_mask must be a 32-bit integer tensor")
        mask_ptr = _ptr(recompute_mask)
    _rc(library().lamp_decode_fwd(
        _f32(q, "q"), _f32(k, "k"), _f32(v, "v"), B, H, Nq, S, D, int(causal), int(mu),
        ctypes.c_float(tau), _f32(out, "out"),
        None if probs is None else _f32(probs, "probs"), mask_ptr,
        ctypes.byref(st) if st is not None else None, ctypes.byref(p)))
    return out, (st.as_dict() if st is not None else None)


MLP_OPS = {"gelu": 1, "layernorm": 2}


def _mlp_params(device, workspace, stage_events, ps_block=0, **opt):
    p = LampParams()
    p.stream = torch.cuda.current_stream(device).cuda_stream
    p.ps_block = int(ps_block)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    for name, t in opt.items():
        if t is not None:
            setattr(p, name, _ptr(t).value)
    if stage_events is not None:
        p.stage_events = stage_events.address
    return p


def _mask_ptr(mask):
    if mask is None:
        return None
    if mask.dtype not in (torch.int32, torch.uint32):
        raise TypeError("recompute_mask must be a 32-bit integer tensor")
    return _ptr(mask)


def _mlp_shapes(x, w):
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    _check(w, "w", tuple(w.shape), (torch.float32,), x.device)
    return x.shape[0], w.shape[0], x.shape[1]


def _mlp_checks(x, M, N, out, recompute_mask, row_err, row_err_lowp, row_count, scores_mix,
                scores_ref, workspace):
    dev = x.device
    f32, f64 = (torch.float32,), (torch.float64,)
    for name, t, shape, dt in (
            ("out", out, (M, N), f32), ("recompute_mask", recompute_mask, (M, (N + 31) // 32),
                                        _INT32),
            ("row_err", row_err, (M,), f64), ("row_err_lowp", row_err_lowp, (M,), f64),
            ("row_count", row_count, (M,), _INT32), ("scores_mix", scores_mix, (M, N), f32),
            ("scores_ref", scores_ref, (M, N), f32)):
        _check(t, name, shape, dt, dev)
    _check_workspace(workspace, dev)


def lamp_mlp_workspace_bytes(M, N, K, op) -> int:
    return int(library().lamp_mlp_workspace_bytes(M, N, K, MLP_OPS.get(op, op)))


def lamp_gemm_scores(x, w, *, mu: int, ylo=None, yref=None):
    """The PS(mu) and FP32 products of x [M, K] and w [N, K] into [M, N]."""
    M, N, K = _mlp_shapes(x, w)
    if ylo is None and yref is None:
        ylo = torch.empty((M, N), device=x.device, dtype=torch.float32)
        yref = torch.empty_like(ylo)
    for name, t in (("ylo", ylo), ("yref", yref)):
        _check(t, name, (M, N), (torch.float32,), x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    _rc(library().lamp_gemm_scores(_f32(x, "x"), _f32(w, "w"), M, N, K, int(mu), _ptr(ylo),
                                      _ptr(yref), stream))
    return ylo, yref


def lamp_gelu_fwd(x, w, *, mu: int, tau: float, out=None, recompute_mask=None,
                  want_stats: bool = True, row_err=None, row_err_lowp=None, row_count=None,
                  scores_mix=None, scores_ref=None, workspace=None, stage_events=None,
                  ps_block: int = 0):
    """GELU(x w^T) with the activation LAMP rule through lamp_gelu_fwd.

    row_err / row_err_lowp (float64 [M]) receive the l1 distances of the LAMP
    and all-PS(mu) outputs to the FP32 one.  Returns (out, stats_or_None).
    """
    M, N, K = _mlp_shapes(x, w)
    if out is None:
        out = torch.empty((M, N), device=x.device, dtype=torch.float32)
    _mlp_checks(x, M, N, out, recompute_mask, row_err, row_err_lowp, row_count, scores_mix,
                scores_ref, workspace)
    p = _mlp_params(x.device, workspace, stage_events, ps_block, row_kl=row_err,
                    row_kl_lowp=row_err_lowp, row_count=row_count, scores_mix=scores_mix,
                    scores_ref=scores_ref)
    st = LampStats() if want_stats else None
    _rc(library().lamp_gelu_fwd(
        _f32(x, "x"), _f32(w, "w"), M, N, K, int(mu), ctypes.c_float(tau), _f32(out, "out"),
        _mask_ptr(recompute_mask), ctypes.byref(st) if st is not None else None, ctypes.byref(p)))
    return out, (st.as_dict() if st is not None else None)


def lamp_layernorm_fwd(x, w, gamma, beta, *, mu: int, eps: float, tau: float, out=None,
                       recompute_mask=None, want_stats: bool = True, row_err=None,
                       row_err_lowp=None, row_count=None, scores_mix=None, scores_ref=None,
                       workspace=None, stage_events=None, ps_block: int = 0):
    """LayerNorm(x w^T) with the greedy LAMP rule through lamp_layernorm_fwd.

    row_err / row_err_lowp (float64 [M]) receive the l2 distances of the LAMP
    and all-PS(mu) outputs to the FP32 one.  Returns (out, stats_or_None).
    """
    M, N, K = _mlp_shapes(x, w)
    if tuple(gamma.shape) != (N,) or tuple(beta.shape) != (N,):
        raise ValueError("gamma and beta must be [N]")
    for name, t in (("gamma", gamma), ("beta", beta)):
        _check(t, name, (N,), (torch.float32,), x.device)
    if out is None:
        out = torch.empty((M, N), device=x.device, dtype=torch.float32)
    _mlp_checks(x, M, N, out, recompute_mask, row_err, row_err_lowp, row_count, scores_mix,
                scores_ref, workspace)
    p = _mlp_params(x.device, workspace, stage_events, ps_block, row_kl=row_err,
                    row_kl_lowp=row_err_lowp, row_count=row_count, scores_mix=scores_mix,
                    scores_ref=scores_ref)
    st = LampStats() if want_stats else None
    _rc(library().lamp_layernorm_fwd(
        _f32(x, "x"), _f32(w, "w"), _f32(gamma, "gamma"), _f32(beta, "beta"), M, N, K, int(mu),
        ctypes.c_float(eps), ctypes.c_float(tau), _f32(out, "out"), _mask_ptr(recompute_mask),
        ctypes.byref(st) if st is not None else None, ctypes.byref(p)))
    return out, (st.as_dict() if st is not None else None)


class HipEvents:
    """hipEvent_t handles for lamp_params.stage_events, via the HIP runtime.

    torch's Event objects create their handle lazily and only see torch's
    streams; the library records these on the stream it was given.  The
    events are timing-only (hipEventDisableSystemFence): a default event's
    record writes back and invalidates the caches, which slows the stage
    after it.  `only`: the stages to time (None: all); the other entries of
    the array are NULL and not recorded.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, n: int, only=None):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                      ctypes.c_uint]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for i in range(n):
            h = ctypes.c_void_p()
            if only is None or i // 2 in only:
                if self._hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                     self.DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles.append(h)
        self.array = (ctypes.c_void_p * n)(*[h.value for h in self.handles])

    @property
    def address(self) -> int:
        return ctypes.cast(self.array, ctypes.c_void_p).value

    def recorded(self, i: int) -> bool:
        return bool(self.handles[i].value) and self._hip.hipEventQuery(self.handles[i]) == 0

    def elapsed_ms(self, a: int, b: int) -> float:
        if not (self.handles[a].value and self.handles[b].value):
            raise RuntimeError("stage not timed (no event created for it)")
        t = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(t), self.handles[a], self.handles[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(t.value)

    def close(self):
        for h in self.handles:
            if h.value:
                self._hip.hipEventDestroy(h)
        self.handles = []

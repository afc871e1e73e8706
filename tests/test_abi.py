"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/lamp.h declares, and rejects bad arguments with the
documented codes before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lamp.h")
LIB = os.path.join(ROOT, "mixed_precision_attention_ps_amd", "liblamp.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixed_precision_attention_ps_amd import build
        build.build()
    from mixed_precision_attention_ps_amd import lamp
    return lamp.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(lamp_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("lamp_attention_fwd", "lamp_attention_fwd_ex", "lamp_workspace_bytes",
                 "lamp_workspace_bytes_ex",
                 "lamp_ps_scores", "lamp_decode_fwd", "lamp_decode_workspace_bytes",
                 "lamp_gelu_fwd", "lamp_layernorm_fwd", "lamp_mlp_workspace_bytes",
                 "lamp_gemm_scores",
                 "lamp_strerror", "lamp_last_error", "lamp_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", "-I",
                        os.path.join(ROOT, "include"), "-"], input='#include "lamp.h"\n',
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


A = 0x10000  # a 16-byte aligned address that is never dereferenced


def call(lib, q=A, k=A, v=A, B=1, H=1, S=8, D=64, causal=0, mu=4, tau=0.1, mode=0, out=A):
    return lib.lamp_attention_fwd(q, k, v, B, H, S, D, causal, mu, ctypes.c_float(tau), mode,
                                  out, None, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(v=None), -1),
    (dict(q=A + 4), -1), (dict(out=A + 8), -1),
    (dict(B=0), -1), (dict(S=0), -1), (dict(D=0), -1), (dict(H=-1), -1),
    (dict(D=6), -2), (dict(D=260), -2),
    (dict(mu=0), -1), (dict(mu=24), -1),
    (dict(tau=float("nan")), -1), (dict(tau=-1.0), -1),
    (dict(causal=2), -1), (dict(mode=3), -1), (dict(mode=-1), -1),
    (dict(mode=1, D=256), -2),
    (dict(B=1 << 20, H=1 << 12, S=4096), -2),
])
def test_invalid_arguments_rejected_before_any_device_call(lib, kw, code):
    rc = call(lib, **kw)
    assert rc == code
    assert lib.lamp_last_error()
    assert lib.lamp_strerror(rc)


def test_ps_scores_argument_checks(lib):
    assert lib.lamp_ps_scores(A, A, 1, 1, 8, 64, 0, 4, None, None, None) == -1
    assert lib.lamp_ps_scores(None, A, 1, 1, 8, 64, 0, 4, A, None, None) == -1
    assert lib.lamp_ps_scores(A, A, 1, 1, 8, 64, 0, 0, A, None, None) == -1
    assert lib.lamp_ps_scores(A, A, 1, 1, 8, 62, 0, 4, A, None, None) == -2


def test_workspace_bytes(lib):
    assert lib.lamp_workspace_bytes(0, 1, 8, 64, 0, 1) == 0
    assert lib.lamp_workspace_bytes(1, 1, 8, 64, 9, 1) == 0
    strict = lib.lamp_workspace_bytes(8, 25, 1024, 64, 0, 1)
    strict_noprobs = lib.lamp_workspace_bytes(8, 25, 1024, 64, 0, 0)
    relaxed = lib.lamp_workspace_bytes(4, 25, 4096, 64, 1, 0)
    # strict keeps the FP32 reference scores and the list: >= 2 * 4 bytes per score
    assert strict >= 8 * 8 * 25 * 1024 * 1024
    assert strict_noprobs >= strict + 4 * 8 * 25 * 1024 * 1024
    # relaxed rows longer than 1024 keys: the bound covers the two-pass form
    # (y^ref and, without probs, y^lo kept dense)
    assert relaxed >= 8 * 4 * 25 * 4096 * 4096



@pytest.mark.parametrize("mode", [0, 2])
def test_long_rows_without_kl_keep_no_reference_scores(lib, mode):
    """Strict rows and the random control past 1024 keys without a row KL:
    the recompute forms each selected score's FP32 dot from the gathered
    query and key rows, so the workspace holds no dense y^ref (one float per
    score less than with the KL)."""
    B, H, S, D = 1, 32, 4096, 64
    with_kl = lib.lamp_workspace_bytes_ex(B, H, S, D, 1, mode, 1, 1, None)
    without = lib.lamp_workspace_bytes_ex(B, H, S, D, 1, mode, 1, 0, None)
    assert 0 < without <= with_kl - 4 * B * H * S * S

def dcall(lib, q=A, k=A, v=A, B=1, H=1, Nq=1, S=8, D=64, causal=1, mu=4, tau=0.1, out=A):
    return lib.lamp_decode_fwd(q, k, v, B, H, Nq, S, D, causal, mu, ctypes.c_float(tau), out,
                               None, None, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(out=None), -1), (dict(v=A + 4), -1),
    (dict(Nq=0), -1), (dict(S=0), -1), (dict(Nq=9, S=8), -1), (dict(Nq=17, S=64), -2),
    (dict(D=6), -2), (dict(D=260), -2), (dict(mu=0), -1), (dict(tau=float("nan")), -1),
    (dict(causal=3), -1), (dict(B=300, H=300), -2),
])
def test_decode_arguments_rejected_before_any_device_call(lib, kw, code):
    rc = dcall(lib, **kw)
    assert rc == code
    assert lib.lamp_last_error()


def test_decode_workspace_bytes(lib):
    assert lib.lamp_decode_workspace_bytes(1, 1, 0, 8, 64) == 0
    assert lib.lamp_decode_workspace_bytes(1, 1, 17, 64, 64) == 0
    ws = lib.lamp_decode_workspace_bytes(8, 25, 4, 16384, 64)
    # y^lo and y^ref per score, the P.V partials (one per 256-key chunk)
    assert ws >= 8 * 8 * 25 * 4 * 16384 + 8 * 8 * 25 * 64 * 4 * 64


def gcall(lib, x=A, w=A, M=4, N=8, K=64, mu=4, tau=0.1, out=A):
    return lib.lamp_gelu_fwd(x, w, M, N, K, mu, ctypes.c_float(tau), out, None, None, None)


def lcall(lib, x=A, w=A, g=A, b=A, M=4, N=8, K=64, mu=4, eps=1e-5, tau=0.1, out=A):
    return lib.lamp_layernorm_fwd(x, w, g, b, M, N, K, mu, ctypes.c_float(eps),
                                  ctypes.c_float(tau), out, None, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(w=None), -1), (dict(out=None), -1), (dict(x=A + 4), -1),
    (dict(M=0), -1), (dict(N=0), -1), (dict(K=0), -1), (dict(K=6), -2),
    (dict(mu=0), -1), (dict(mu=24), -1), (dict(tau=float("nan")), -1), (dict(tau=-0.5), -1),
    (dict(M=1 << 30, N=1 << 30), -2), (dict(M=1, K=1 << 26), -2),
])
def test_gelu_arguments_rejected_before_any_device_call(lib, kw, code):
    assert gcall(lib, **kw) == code
    assert lib.lamp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), -1), (dict(b=None), -1), (dict(eps=-1.0), -1), (dict(eps=float("nan")), -1),
    (dict(N=8193), -2), (dict(K=10), -2), (dict(mu=30), -1), (dict(M=0), -1),
])
def test_layernorm_arguments_rejected_before_any_device_call(lib, kw, code):
    assert lcall(lib, **kw) == code
    assert lib.lamp_last_error()


def test_gemm_scores_argument_checks(lib):
    assert lib.lamp_gemm_scores(A, A, 4, 8, 64, 4, None, None, None) == -1
    assert lib.lamp_gemm_scores(None, A, 4, 8, 64, 4, A, None, None) == -1
    assert lib.lamp_gemm_scores(A, A, 4, 8, 62, 4, A, None, None) == -2
    assert lib.lamp_gemm_scores(A, A, 4, 8, 64, 0, A, None, None) == -1


def test_mlp_workspace_bytes(lib):
    assert lib.lamp_mlp_workspace_bytes(0, 8, 64, 1) == 0
    assert lib.lamp_mlp_workspace_bytes(4, 8, 64, 0) == 0
    assert lib.lamp_mlp_workspace_bytes(4, 9000, 64, 2) == 0
    M, N = 1024, 6400
    gelu = lib.lamp_mlp_workspace_bytes(M, N, 1600, 1)
    # per-(row, 64-column tile) error partials, the mask, per-row outputs
    assert gelu >= 16 * M * (N // 64) + 4 * M * (N // 32) + 20 * M
    ln = lib.lamp_mlp_workspace_bytes(M, 1600, 6400, 2)
    # y^lo and y^ref of the whole product
    assert ln >= 8 * M * 1600


def test_ps_block_checked_before_any_device_call(lib):
    from mixed_precision_attention_ps_amd import lamp
    for b, code in ((-1, -1), (2, -2), (3, -2), (6, -2), (12, -2), (1 << 25, -2)):
        p = lamp.LampParams()
        p.ps_block = b
        rc = lib.lamp_attention_fwd_ex(A, A, A, 1, 1, 8, 64, 0, 4, ctypes.c_float(0.1), 0, A,
                                       None, None, None, ctypes.byref(p))
        assert rc == code, (b, rc)
        rc = lib.lamp_decode_fwd(A, A, A, 1, 1, 1, 8, 64, 1, 4, ctypes.c_float(0.1), A, None,
                                 None, None, ctypes.byref(p))
        assert rc == code, (b, rc)
        rc = lib.lamp_gelu_fwd(A, A, 4, 8, 64, 4, ctypes.c_float(0.1), A, None, None,
                               ctypes.byref(p))
        assert rc == code, (b, rc)


def test_relaxed_path_checked_before_any_device_call(lib):
    from mixed_precision_attention_ps_amd import lamp
    for rp in (-1, 3, 100):
        p = lamp.LampParams()
        p.relaxed_path = rp
        rc = lib.lamp_attention_fwd_ex(A, A, A, 1, 1, 8, 64, 0, 4, ctypes.c_float(0.1), 1, A,
                                       None, None, None, ctypes.byref(p))
        assert rc == -1, (rp, rc)


def test_workspace_covers_both_relaxed_paths(lib):
    # rows of <= 1024 keys: the two-pass relaxed path keeps per-tile partials
    # (24 bytes per row and tile) and, without probs, the score rows
    B, H, S = 8, 25, 1024
    rows, tiles = B * H * S, S // 64
    with_probs = lib.lamp_workspace_bytes(B, H, S, 64, 1, 1)
    no_probs = lib.lamp_workspace_bytes(B, H, S, 64, 1, 0)
    assert with_probs >= 24 * rows * tiles
    assert no_probs >= 4 * rows * S + 24 * rows * tiles


def test_workspace_covers_relaxed_long_rows_two_pass(lib):
    # rows longer than 1024 keys in two passes: y^ref, per-tile partials and
    # per-row statistics, and without probs the score rows too
    B, H, S = 4, 25, 4096
    rows, tiles = B * H * S, S // 64
    with_probs = lib.lamp_workspace_bytes(B, H, S, 64, 1, 1)
    no_probs = lib.lamp_workspace_bytes(B, H, S, 64, 1, 0)
    assert with_probs >= 4 * rows * S + 24 * rows * tiles
    assert no_probs >= 8 * rows * S + 24 * rows * tiles


def test_workspace_bytes_ex(lib):
    from mixed_precision_attention_ps_amd import lamp
    ex = lamp.lamp_workspace_bytes_ex
    B, H, S = 4, 25, 4096
    rows, scores = B * H * S, B * H * S * S
    # the fused one-pass relaxed kernel keeps per-row state only
    fused = lamp.LampParams()
    fused.relaxed_path = 1
    assert ex(B, H, S, 64, 1, "relaxed", 1, 1, fused) < 64 * rows
    # the two-pass form (the default for these rows when it fits): y^ref,
    # partials, row statistics; y^lo too when neither probs nor scores_mix
    two = ex(B, H, S, 64, 1, "relaxed", 1, 1, None)
    assert two >= 4 * scores + 24 * rows * (S // 64)
    assert ex(B, H, S, 64, 1, "relaxed", 0, 1, None) >= two + 4 * scores
    # every exact size is within the upper bound
    for mode in ("strict", "relaxed", "random"):
        for probs in (0, 1):
            for S_ in (512, 1024, 2048):
                for causal in (0, 1):
                    for rp in (0, 1, 2):
                        p = lamp.LampParams()
                        p.relaxed_path = rp
                        e = ex(2, 3, S_, 64, causal, mode, probs, 1, p)
                        assert 0 < e <= lib.lamp_workspace_bytes(2, 3, S_, 64,
                                                                 lamp.MODES[mode], probs)
    # caller-passed buffers leave the workspace
    p = lamp.LampParams()
    p.relaxed_path = 2
    with_ref = ex(B, H, S, 64, 1, "relaxed", 1, 1, p)
    p.scores_ref = 256
    assert ex(B, H, S, 64, 1, "relaxed", 1, 1, p) <= with_ref - 4 * scores
    # invalid arguments give 0
    assert ex(0, H, S, 64, 1, "relaxed", 1, 1, None) == 0
    assert ex(B, H, S, 64, 2, "relaxed", 1, 1, None) == 0
    assert ex(B, H, S, 256, 1, "relaxed", 1, 1, None) == 0
    bad = lamp.LampParams()
    bad.relaxed_path = 3
    assert ex(B, H, S, 64, 1, "relaxed", 1, 1, bad) == 0


def test_version_and_strerror(lib):
    assert lib.lamp_version() >= 10000
    assert lib.lamp_strerror(0) == b"success"
    assert lib.lamp_strerror(-4) == b"out of device memory"


def test_block_k_checked_before_any_device_call(lib):
    """The relaxed rule's block width: 0 (the default) and 64 are the
    implemented width; anything else is refused in relaxed mode and in the
    decode entry point (both apply the relaxed rule)."""
    from mixed_precision_attention_ps_amd import lamp
    for b, code in ((-1, -1), (32, -2), (128, -2), (1, -2)):
        p = lamp.LampParams()
        p.block_k = b
        rc = lib.lamp_attention_fwd_ex(A, A, A, 1, 1, 8, 64, 0, 4, ctypes.c_float(0.1), 1, A,
                                       None, None, None, ctypes.byref(p))
        assert rc == code, (b, rc)
        assert b"block_k" in lib.lamp_last_error()
        rc = lib.lamp_decode_fwd(A, A, A, 1, 1, 1, 8, 64, 1, 4, ctypes.c_float(0.1), A, None,
                                 None, None, ctypes.byref(p))
        assert rc == code, (b, rc)
        assert lamp.lamp_workspace_bytes_ex(1, 1, 8, 64, 1, "relaxed", 1, 1, p) == 0
    p = lamp.LampParams()
    p.block_k = 64
    assert lamp.lamp_workspace_bytes_ex(1, 1, 8, 64, 1, "relaxed", 1, 1, p) > 0
    # other modes ignore it
    p.block_k = 32
    assert lamp.lamp_workspace_bytes_ex(1, 1, 8, 64, 1, "strict", 1, 1, p) > 0


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes structures have the C layout of include/lamp.h."""
    from mixed_precision_attention_ps_amd import lamp
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "lamp.h"\n'
        "#define F(T, f) printf(#T \" \" #f \" %zu\\n\", offsetof(T, f))\n"
        "int main(void) {\n"
        ' printf("lamp_stats size %zu\\n", sizeof(lamp_stats));\n'
        ' printf("lamp_params size %zu\\n", sizeof(lamp_params));\n'
        + "".join(f" F(lamp_stats, {n});\n" for n, _ in lamp.LampStats._fields_)
        + "".join(f" F(lamp_params, {n});\n" for n, _ in lamp.LampParams._fields_)
        + " return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        t, f, v = line.split()
        got[(t, f)] = int(v)
    assert got[("lamp_stats", "size")] == ctypes.sizeof(lamp.LampStats)
    assert got[("lamp_params", "size")] == ctypes.sizeof(lamp.LampParams)
    for cls, t in ((lamp.LampStats, "lamp_stats"), (lamp.LampParams, "lamp_params")):
        for n, _ in cls._fields_:
            assert got[(t, n)] == getattr(cls, n).offset, (t, n)


def test_last_impl_before_any_call(lib):
    # a fresh thread has run nothing
    import threading
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.lamp_last_impl()))
    th.start()
    th.join()
    assert seen == [0]


def _meta(*shape, dtype=None):
    import torch
    return torch.empty(shape, device="meta", dtype=dtype or torch.float32)


@pytest.mark.parametrize("name,bad", [
    ("k", lambda t: _meta(1, 2, 8, 32)), ("v", lambda t: _meta(1, 2, 9, 64)),
    ("out", lambda t: _meta(1, 2, 8, 64, dtype=t.float64)),
    ("probs", lambda t: _meta(1, 2, 8, 9)), ("probs", lambda t: _meta(1, 2, 64)),
    ("recompute_mask", lambda t: _meta(1, 2, 8, 2, dtype=t.int32)),
    ("recompute_mask", lambda t: _meta(1, 2, 8, 1, dtype=t.float32)),
    ("row_kl", lambda t: _meta(1, 2, 8)), ("row_kl_lowp", lambda t: _meta(1, 2, 9, dtype=t.float64)),
    ("row_count", lambda t: _meta(1, 2, 8, dtype=t.int64)),
    ("scores_mix", lambda t: _meta(1, 2, 8, 7)), ("scores_ref", lambda t: _meta(2, 2, 8, 8)),
    ("workspace", lambda t: t.empty(64, dtype=t.uint8)),
])
def test_binding_refuses_mismatched_tensors(name, bad):
    """Every tensor the attention binding hands to the library is checked for
    shape, dtype and device first (a wrong size would let the kernels run past
    its allocation); a refused call never reaches the library."""
    import torch
    from mixed_precision_attention_ps_amd import lamp
    q = _meta(1, 2, 8, 64)
    kw = {name: bad(torch)}
    args = dict(k=_meta(1, 2, 8, 64), v=_meta(1, 2, 8, 64))
    args.update({k_: v_ for k_, v_ in kw.items() if k_ in ("k", "v")})
    rest = {k_: v_ for k_, v_ in kw.items() if k_ not in ("k", "v")}
    with pytest.raises((ValueError, TypeError)):
        lamp.lamp_attention_fwd(q, args["k"], args["v"], causal=True, mu=4, tau=0.1, **rest)


@pytest.mark.parametrize("name,bad", [
    ("out", lambda t: _meta(1, 2, 3, 64)), ("probs", lambda t: _meta(1, 2, 2, 100)),
    ("recompute_mask", lambda t: _meta(1, 2, 2, 4, dtype=t.int32)),
    ("row_kl", lambda t: _meta(1, 2, 2)), ("row_count", lambda t: _meta(1, 2, 1, dtype=t.int32)),
    ("scores_ref", lambda t: _meta(1, 2, 2, 64)),
])
def test_decode_binding_refuses_mismatched_tensors(name, bad):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    q, k, v = _meta(1, 2, 2, 64), _meta(1, 2, 96, 64), _meta(1, 2, 96, 64)
    with pytest.raises((ValueError, TypeError)):
        lamp.lamp_decode_fwd(q, k, v, causal=True, mu=4, tau=0.1, **{name: bad(torch)})


@pytest.mark.parametrize("name,bad", [
    ("out", lambda t: _meta(4, 9)), ("recompute_mask", lambda t: _meta(4, 2, dtype=t.int32)),
    ("row_err", lambda t: _meta(4)), ("row_count", lambda t: _meta(5, dtype=t.int32)),
    ("scores_mix", lambda t: _meta(8, 4)),
])
def test_mlp_binding_refuses_mismatched_tensors(name, bad):
    import torch
    from mixed_precision_attention_ps_amd import lamp
    x, w = _meta(4, 64), _meta(8, 64)
    with pytest.raises((ValueError, TypeError)):
        lamp.lamp_gelu_fwd(x, w, mu=4, tau=0.1, **{name: bad(torch)})
    with pytest.raises((ValueError, TypeError)):
        lamp.lamp_layernorm_fwd(x, w, _meta(8), _meta(8), mu=4, eps=1e-5, tau=0.1,
                                **{name: bad(torch)})


def test_noalloc_checks_before_any_device_call(lib):
    """lamp_attention_fwd_noalloc refuses a workspace and any call whose
    scratch need exceeds its fixed array, before touching the GPU."""
    from mixed_precision_attention_ps_amd import lamp
    p = lamp.LampParams()
    p.workspace = 1 << 20
    p.workspace_bytes = 1 << 20
    rc = lib.lamp_attention_fwd_noalloc(A, A, A, 1, 1, 8, 64, 0, 4, ctypes.c_float(0.1), 0, A,
                                        None, None, None, ctypes.byref(p))
    assert rc == -1 and b"workspace" in lib.lamp_last_error()
    # the GPT-2-XL layer without caller buffers: y^lo, y^ref and partials
    # (about 1.8 GB) do not fit 64 MiB
    need = lamp.lamp_workspace_bytes_ex(8, 25, 1024, 64, 1, "strict", 0, 1, None)
    assert need > (64 << 20)
    rc = lib.lamp_attention_fwd_noalloc(A, A, A, 8, 25, 1024, 64, 1, 4, ctypes.c_float(0.1), 0,
                                        A, None, None, ctypes.byref(lamp.LampStats()), None)
    assert rc == -2 and b"scratch" in lib.lamp_last_error()
    # argument checks come first, as for the other entry points
    rc = lib.lamp_attention_fwd_noalloc(None, A, A, 1, 1, 8, 64, 0, 4, ctypes.c_float(0.1), 0,
                                        A, None, None, None, None)
    assert rc == -1

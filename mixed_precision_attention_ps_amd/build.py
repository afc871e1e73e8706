"""Build the LAMP HIP library (liblamp.so) for gfx950 with hipcc.

Every source is compiled to an object (in parallel) and linked into
``mixed_precision_attention_ps_amd/liblamp.so``.  Flags that matter for the
numerics:
  -ffp-contract=off   keep every FP32 multiply and add separately rounded
                      (HIP's device default would fuse them into FMAs);
  packed-fp32-ops off plain scalar FP32 instructions only.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblamp.so")
ARCH = os.environ.get("LAMP_OFFLOAD_ARCH", "gfx950")

SOURCES = ["scores.hip", "select.hip", "rows.hip", "finish.hip", "relaxed.hip", "decode.hip",
           "mlp.hip", "lamp_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", *COMMON, *extra, "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        msgs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def asm(src: str) -> str:
    """Device assembly of one source (for inspection of the hot loop)."""
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".s")
    os.makedirs(OBJ, exist_ok=True)
    cmd = [hipcc(), "-S", *COMMON, "--offload-device-only", "-x", "hip",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)

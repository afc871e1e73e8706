"""CPU-side test helpers written in C (compiled with gcc on first use).

``rn_bits_check.c`` -- an integer formulation of RN_mu on FP32 bit patterns,
used to sweep the oracle's rounding exhaustively.
``fast_ps_emul.c``  -- a scalar CPU emulation of the FP32 instruction
sequence the GPU kernels use for PS(mu) products and sums; checked against
the oracle on the CPU so that the kernels' arithmetic premise is tested
before any GPU run.  It is test code: the product never links it.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")


def load(name: str):
    src = os.path.join(_HERE, name + ".c")
    os.makedirs(_BUILD, exist_ok=True)
    so = os.path.join(_BUILD, "lib" + name + ".so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        "-std=c11", "-Wall", "-fPIC", "-shared", "-o", tmp, src, "-lm"],
                       check=True)
        os.replace(tmp, so)
    return ctypes.CDLL(so)

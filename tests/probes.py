"""Build and load the test-only GPU probe library (tests/fp4_scan.hip -> tests/_build/).

It is compiled by ``__graft_entry__.build()`` together with the product library, with the
same hipcc flags, so that GPU test runs only load it. The product library never loads it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libfp4scan.so")
SRC = os.path.join(HERE, "fp4_scan.hip")


def build(verbose: bool = False) -> str:
    from dual_scale_w4a4_amd import build as dq_build

    os.makedirs(BUILD, exist_ok=True)
    cmd = [dq_build.hipcc(), *dq_build.HIPCC_FLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed building the FP4 scan probe:\n" + res.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib() -> ctypes.CDLL:
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB)
    P, I, U, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_float
    L.fp4_scan.argtypes = [I, F, U, P, I, P]
    L.fp4_scan.restype = I
    L.fp4_decode.argtypes = [F, P, P]
    L.fp4_decode.restype = I
    L.fp4_encode.argtypes = [F, P, P, I, P]
    L.fp4_encode.restype = I
    return L

"""CPU oracle for the DualQuant dual-scale solver (ctypes wrapper of ``libdq_ref.so``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It never touches the
HIP library and the HIP library never touches it; they share only the seeded
input generators in ``workloads``.

The C source (``dq_ref.c``) is a plain double-precision reading of the method
on the DualQuant pages (daiwk reproduction notes, "核心公式" eq. 1-2 and the
conventions under them; trove summary, "How it works"). Every function it
exports is pinned by ``tests/test_oracle_*.py`` against brute force, library
routines, closed forms and invariants, not against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DQ_REF_LIB: load another build of the same source instead (the planted-mistake tests run
# the pins against deliberately broken copies of dq_ref.c built in a scratch directory)
LIB_PATH = os.environ.get("DQ_REF_LIB") or os.path.join(_HERE, "libdq_ref.so")

FMT = {"int4_bf16": 0, "mxint4": 1, "mxfp4": 2, "nvfp4": 3}
DTYPE = {"f32": 0, "bf16": 1}
STATUS = {0: "OK", 1: "ERR_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_NONFINITE", 4: "ERR_RANGE",
          7: "ERR_INTERNAL"}


GCC_FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    """Compile libdq_ref.so with gcc (plain C11, -O2, no FMA contraction, OpenMP)."""
    if os.environ.get("DQ_REF_LIB"):
        raise RuntimeError("DQ_REF_LIB names a prebuilt oracle library; not rebuilding it")
    cmd = ["gcc", *GCC_FLAGS, os.path.join(_HERE, "dq_ref.c"), "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    global _lib
    _lib = None
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) and not os.environ.get("DQ_REF_LIB"):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.dq_ref_quantize.argtypes = [P, I, I64, I64, I, I, P, P, P, P, P]
        L.dq_ref_quantize.restype = I
        L.dq_ref_quantize_act.argtypes = [P, I, I64, I64, I, I, P, P, P, P]
        L.dq_ref_solve_pass_g.argtypes = [P, I, I64, I64, I, I, P, P, P, P, P, P, P, P]
        L.dq_ref_solve_pass_g.restype = I
        L.dq_ref_gemm_mx.argtypes = [P, P, I64, I64, P, P, I64, P, P]
        L.dq_ref_gemm_mx.restype = I
        L.dq_ref_quantize_act.restype = I
        L.dq_ref_solve.argtypes = [P, I, I64, I64, I, I, I, P, P, F, P, P, P, P, P, P]
        L.dq_ref_solve.restype = I
        L.dq_ref_solve_diag.argtypes = [P, I, I64, I64, I, I, I, P, P, F, P, P, P, P, P, P, P, P]
        L.dq_ref_solve_diag.restype = I
        for name in ("dq_ref_project", "dq_ref_proj_margin"):
            getattr(L, name).argtypes = [I, D]
            getattr(L, name).restype = D
        for name in ("dq_ref_bf16_rne", "dq_ref_e4m3_rne_sat", "dq_ref_e2m1_round"):
            getattr(L, name).argtypes = [D]
            getattr(L, name).restype = D
        L.dq_ref_set_threads.argtypes = [I]
        L.dq_ref_set_threads.restype = I
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status} ({STATUS.get(status, '?')})")
        self.status = status


def _ptr(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _prep_w(W: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    W = np.ascontiguousarray(W)
    if W.dtype != want:
        raise TypeError(f"W must be {want} for dtype {dtype}")
    return W


def _scale_dtype(fmt: str):
    return np.uint16 if fmt == "int4_bf16" else np.uint8


def set_threads(n: int) -> int:
    return int(lib().dq_ref_set_threads(int(n)))


def quantize(W: np.ndarray, dtype: str, fmt: str, group: int, a=None, b=None,
             g: float = 0.0) -> Dict[str, np.ndarray]:
    """One Q pass on X(a, b). Returns codes (rows x cols/2 u8), scales, g."""
    W = _prep_w(W, dtype)
    rows, cols = W.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // group), _scale_dtype(fmt))
    a = None if a is None else np.ascontiguousarray(a, np.float32)
    b = None if b is None else np.ascontiguousarray(b, np.float32)
    gbuf = np.array([g], np.float32)
    st = lib().dq_ref_quantize(_ptr(W), DTYPE[dtype], rows, cols, FMT[fmt], group, _ptr(a),
                               _ptr(b), _ptr(gbuf), _ptr(codes), _ptr(scales))
    if st:
        raise OracleError(st)
    return {"codes": codes, "scales": scales, "g": float(gbuf[0])}


def quantize_act(X: np.ndarray, dtype: str, fmt: str, group: int, b=None,
                 g: float = 0.0) -> Dict[str, np.ndarray]:
    """Activation quantization: Q of x = fl32(X * b) per row (tokens x cols), groups along
    the channels. Returns codes (tokens x cols/2 u8), scales, g."""
    X = _prep_w(X, dtype)
    rows, cols = X.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // group), _scale_dtype(fmt))
    b = None if b is None else np.ascontiguousarray(b, np.float32)
    gbuf = np.array([g], np.float32)
    st = lib().dq_ref_quantize_act(_ptr(X), DTYPE[dtype], rows, cols, FMT[fmt], group, _ptr(b),
                                   _ptr(gbuf), _ptr(codes), _ptr(scales))
    if st:
        raise OracleError(st)
    return {"codes": codes, "scales": scales, "g": float(gbuf[0])}


def gemm_mx(act_codes, act_scales, w_codes, w_scales, a=None) -> np.ndarray:
    """W4A4 product of MXFP4 activations and weights (codes and E8M0 scales as the quantizers
    return them) with the weights' row scales a: tokens x out float64."""
    act_codes = np.ascontiguousarray(act_codes, np.uint8)
    act_scales = np.ascontiguousarray(act_scales, np.uint8)
    w_codes = np.ascontiguousarray(w_codes, np.uint8)
    w_scales = np.ascontiguousarray(w_scales, np.uint8)
    tokens, K = act_codes.shape[0], act_codes.shape[1] * 2
    out = w_codes.shape[0]
    a = None if a is None else np.ascontiguousarray(a, np.float32)
    Y = np.zeros((tokens, out), np.float64)
    st = lib().dq_ref_gemm_mx(_ptr(act_codes), _ptr(act_scales), tokens, K, _ptr(w_codes),
                              _ptr(w_scales), out, _ptr(a), _ptr(Y))
    if st:
        raise OracleError(st)
    return Y


def solve_pass_g(W: np.ndarray, dtype: str, group: int, T: int, a0=None,
                 b0=None) -> Dict[str, np.ndarray]:
    """NVFP4 solve with the tensor scale recomputed before every Q pass."""
    W = _prep_w(W, dtype)
    rows, cols = W.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // group), np.uint8)
    a = np.zeros(rows, np.float32)
    b = np.zeros(cols, np.float32)
    mse = np.zeros(T + 1, np.float64)
    g = np.zeros(1, np.float32)
    a0 = None if a0 is None else np.ascontiguousarray(a0, np.float32)
    b0 = None if b0 is None else np.ascontiguousarray(b0, np.float32)
    st = lib().dq_ref_solve_pass_g(_ptr(W), DTYPE[dtype], rows, cols, group, T, _ptr(a0),
                                   _ptr(b0), _ptr(codes), _ptr(scales), _ptr(g), _ptr(a), _ptr(b),
                                   _ptr(mse))
    if st:
        raise OracleError(st)
    return {"codes": codes, "scales": scales, "g": float(g[0]), "a": a, "b": b, "mse": mse}


def solve(W: np.ndarray, dtype: str, fmt: str, group: int, T: int, a0=None, b0=None,
          g0: float = 0.0, diag: bool = False) -> Dict[str, np.ndarray]:
    """T iterations of the dual-scale block-coordinate descent."""
    W = _prep_w(W, dtype)
    rows, cols = W.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // group), _scale_dtype(fmt))
    a = np.zeros(rows, np.float32)
    b = np.zeros(cols, np.float32)
    mse = np.zeros(T + 1, np.float64)
    g = np.zeros(1, np.float32)
    a0 = None if a0 is None else np.ascontiguousarray(a0, np.float32)
    b0 = None if b0 is None else np.ascontiguousarray(b0, np.float32)
    changes = np.zeros(4 * max(T, 1), np.int64) if diag else None
    margin = np.zeros(2 * max(T, 1), np.float64) if diag else None
    st = lib().dq_ref_solve_diag(_ptr(W), DTYPE[dtype], rows, cols, FMT[fmt], group, T,
                                 _ptr(a0), _ptr(b0), float(g0), _ptr(codes), _ptr(scales),
                                 _ptr(g), _ptr(a), _ptr(b), _ptr(mse), _ptr(changes),
                                 _ptr(margin))
    if st:
        raise OracleError(st)
    out = {"codes": codes, "scales": scales, "g": float(g[0]), "a": a, "b": b, "mse": mse}
    if diag:
        out["changes"] = changes[: 4 * T].reshape(T, 4)
        out["margin"] = margin[: 2 * T].reshape(T, 2)
    return out


def project(fmt: str, v: float) -> float:
    return float(lib().dq_ref_project(FMT[fmt], float(v)))


def proj_margin(fmt: str, v: float) -> float:
    """Relative distance from v to the nearest decision point of the projection."""
    return float(lib().dq_ref_proj_margin(FMT[fmt], float(v)))


def bf16_rne(v: float) -> float:
    return float(lib().dq_ref_bf16_rne(float(v)))


def e4m3_rne_sat(v: float) -> float:
    return float(lib().dq_ref_e4m3_rne_sat(float(v)))


def e2m1_round(v: float) -> float:
    return float(lib().dq_ref_e2m1_round(float(v)))

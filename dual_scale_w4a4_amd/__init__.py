"""Python binding of libdq.so, the MI355X dual-scale weight-reconstruction solver.

Argument marshalling only: every step of the solver runs in the HIP kernels behind the C ABI
declared in include/dq.h. PyTorch provides device memory and the current stream. There is
no CPU fallback: if libdq.so is missing or no GPU is present, calls raise.

    import dual_scale_w4a4_amd as dq
    out = dq.solve(W_cuda_bf16, "mxfp4", group=32, T=20)
    out["codes"], out["scales"], out["a"], out["b"], out["mse"], out["g"]
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dq.h")

FMT = {"int4_bf16": 0, "mxint4": 1, "mxfp4": 2, "nvfp4": 3}
DTYPE = {"f32": 0, "bf16": 1}
STATUS = {0: "DQ_OK", 1: "DQ_ERR_ARG", 2: "DQ_ERR_UNSUPPORTED", 3: "DQ_ERR_NONFINITE",
          4: "DQ_ERR_RANGE", 5: "DQ_ERR_WORKSPACE", 6: "DQ_ERR_HIP", 7: "DQ_ERR_INTERNAL"}
SOLVE_TWO_SWEEP = 1
SOLVE_PER_PASS_G = 2
KERNEL_KINDS = ("setup", "fused", "row", "col", "final", "emit", "rowres")


class DQError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class _Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 7), ("launches", ctypes.c_int64 * 7),
                ("used_fused", ctypes.c_int), ("isolated_ms", ctypes.c_double),
                ("isolated_launches", ctypes.c_int), ("flush", ctypes.c_void_p),
                ("flush_bytes", ctypes.c_size_t), ("cold_ms", ctypes.c_double),
                ("warm_ms", ctypes.c_double), ("per_launch", ctypes.c_int)]


class _Init(ctypes.Structure):
    _fields_ = [("a0", ctypes.c_void_p), ("b0", ctypes.c_void_p), ("g0", ctypes.c_float),
                ("flags", ctypes.c_uint)]


class _Shape(ctypes.Structure):
    """dq_launch_shape (include/dq_bench.h): 0 keeps a field's default."""
    _fields_ = [("fused_halves", ctypes.c_int), ("fused_step_rows", ctypes.c_int),
                ("fused_target", ctypes.c_int), ("pass_target", ctypes.c_int),
                ("sweep_target", ctypes.c_int), ("row_resident", ctypes.c_int),
                ("rowres_target", ctypes.c_int), ("fused_ahead", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdq.so (built by dual_scale_w4a4_amd.build); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m dual_scale_w4a4_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.dq_workspace_bytes.argtypes = [I64, I64, I, I]
        L.dq_workspace_bytes.restype = SZ
        L.dq_solve.argtypes = [P, I, I64, I64, I, I, I, ctypes.POINTER(_Init), P, P, P, P, P, P,
                               P, SZ, P]
        L.dq_solve.restype = I
        L.dq_solve_timed.argtypes = [P, I, I64, I64, I, I, I, ctypes.POINTER(_Init), P, P, P, P,
                                     P, P, P, SZ, ctypes.POINTER(_Shape), ctypes.POINTER(_Timing),
                                     P]
        L.dq_solve_timed.restype = I
        L.dq_bench_workspace_bytes.argtypes = [I64, I64, I, I, ctypes.POINTER(_Shape)]
        L.dq_bench_workspace_bytes.restype = SZ
        L.dq_bench_fp4_mfma_rate.argtypes = [I, P, ctypes.POINTER(ctypes.c_double)]
        L.dq_bench_fp4_mfma_rate.restype = I
        L.dq_quantize.argtypes = [P, I, I64, I64, I, I, P, P, P, P, P, P, SZ, P]
        L.dq_quantize.restype = I
        L.dq_act_workspace_bytes.argtypes = [I64, I64, I, I]
        L.dq_act_workspace_bytes.restype = SZ
        L.dq_quantize_act.argtypes = [P, I, I64, I64, I, I, P, ctypes.c_float, P, P, P, P, SZ, P]
        L.dq_quantize_act.restype = I
        L.dq_quantize_act_async.argtypes = [P, I, I64, I64, I, I, P, ctypes.c_float, P, P, P, P,
                                            P, SZ, P]
        L.dq_quantize_act_async.restype = I
        L.dq_solve_async.argtypes = [P, I, I64, I64, I, I, I, ctypes.POINTER(_Init), P, P, P, P, P,
                                     P, P, P, SZ, P]
        L.dq_solve_async.restype = I
        L.dq_solve_async_noalloc.argtypes = [P, I, I64, I64, I, I, I, ctypes.POINTER(_Init), P, P,
                                             P, P, P, P, P, P]
        L.dq_solve_async_noalloc.restype = I
        L.dq_gemm_mx.argtypes = [P, P, I64, I64, P, P, P, I64, I, P, P]
        L.dq_gemm_mx.restype = I
        L.dq_gemm_pack_bytes.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        L.dq_gemm_pack_bytes.restype = I
        L.dq_gemm_pack_weights.argtypes = [P, P, I64, I64, P, P, P]
        L.dq_gemm_pack_weights.restype = I
        L.dq_gemm_mx_packed.argtypes = [P, P, I64, I64, P, P, P, I64, I, P, P]
        L.dq_gemm_mx_packed.restype = I
        L.dq_status_str.argtypes = [I]
        L.dq_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().dq_status_str(int(status)).decode()


def workspace_bytes(rows: int, cols: int, fmt: str, group: int) -> int:
    return int(lib().dq_workspace_bytes(int(rows), int(cols), FMT[fmt], int(group)))


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_w(W):
    torch = _torch()
    if not W.is_cuda:
        raise ValueError("W must be a CUDA (HIP) tensor")
    if W.dtype not in (torch.float32, torch.bfloat16) or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D float32 or bfloat16 tensor")
    return "bf16" if W.dtype == torch.bfloat16 else "f32"


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _outputs(W, fmt, group):
    torch = _torch()
    rows, cols = W.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=W.device)
    sdt = torch.int16 if fmt == "int4_bf16" else torch.uint8
    scales = torch.empty((rows, cols // group), dtype=sdt, device=W.device)
    return codes, scales


def _vec(v, n, device):
    torch = _torch()
    if v is None:
        return None
    v = torch.as_tensor(v, dtype=torch.float32, device=device).contiguous()
    if v.numel() != n:
        raise ValueError("scale vector has the wrong length")
    return v


def solve(W, fmt: str, group: int, T: int, a0=None, b0=None, g0: float = 0.0,
          two_sweep: bool = False, workspace=None, timing: bool = False,
          stream=None, flush=None, per_pass_g: bool = False, shape=None) -> Dict[str, object]:
    """dq_solve on W (rows x cols, CUDA float32 / bfloat16). Returns a dict of device
    tensors codes (rows x cols/2 u8), scales (rows x cols/group; int16 holding bf16 bits for
    int4_bf16, else u8), a, b (float32), mse (T+1 float64), g (float32[1]).

    ``timing`` or ``shape`` (a dict of dq_launch_shape fields) go through the measurement
    entry point dq_solve_timed (include/dq_bench.h), which adds per-kernel-kind milliseconds
    and launch counts, whether the single-sweep path was used, and the isolated and cold /
    warm re-runs of its pass (``flush``: a device buffer read in full before each cold
    re-run)."""
    torch = _torch()
    dt = _check_w(W)
    rows, cols = W.shape
    dev = W.device
    codes, scales = _outputs(W, fmt, group)
    a = torch.empty(rows, dtype=torch.float32, device=dev)
    b = torch.empty(cols, dtype=torch.float32, device=dev)
    mse = torch.empty(T + 1, dtype=torch.float64, device=dev)
    g = torch.zeros(1, dtype=torch.float32, device=dev)
    a0 = _vec(a0, rows, dev)
    b0 = _vec(b0, cols, dev)
    flags = (SOLVE_TWO_SWEEP if two_sweep else 0) | (SOLVE_PER_PASS_G if per_pass_g else 0)
    init = _Init(_ptr(a0), _ptr(b0), float(g0), flags)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    args = (W.data_ptr(), DTYPE[dt], rows, cols, FMT[fmt], group, T, ctypes.byref(init),
            codes.data_ptr(), scales.data_ptr(), g.data_ptr(), a.data_ptr(), b.data_ptr(),
            mse.data_ptr(), ws_ptr, ws_bytes)
    tm = None
    if timing or shape is not None:
        tm = _Timing()
        if flush is not None:
            tm.flush = flush.data_ptr()
            tm.flush_bytes = flush.numel() * flush.element_size() // 16 * 16
        sh = _Shape(**(shape or {}))
        st = lib().dq_solve_timed(*args, ctypes.byref(sh), ctypes.byref(tm), _stream(stream))
    else:
        st = lib().dq_solve(*args, _stream(stream))
    if st != 0:
        raise DQError(st, "dq_solve")
    out = {"codes": codes, "scales": scales, "a": a, "b": b, "mse": mse, "g": g}
    if tm is not None:
        out["timing"] = {k: (tm.ms[i], tm.launches[i]) for i, k in enumerate(KERNEL_KINDS)}
        out["used_fused"] = bool(tm.used_fused)
        out["isolated"] = (tm.isolated_ms, tm.isolated_launches)
        out["cold_warm"] = (tm.cold_ms, tm.warm_ms, tm.per_launch)
    return out


def bench_workspace_bytes(rows: int, cols: int, fmt: str, group: int, shape=None) -> int:
    """dq_bench_workspace_bytes: the workspace of a solve in a given launch shape."""
    sh = _Shape(**(shape or {}))
    return int(lib().dq_bench_workspace_bytes(int(rows), int(cols), FMT[fmt], int(group),
                                              ctypes.byref(sh)))


def bench_fp4_mfma_rate(iters: int = 20000, stream=None) -> float:
    """dq_bench_fp4_mfma_rate: the attainable dense-equivalent TFLOP/s of the scaled FP4 matrix
    instruction (register operands only)."""
    out = ctypes.c_double(0.0)
    st = lib().dq_bench_fp4_mfma_rate(int(iters), _stream(stream), ctypes.byref(out))
    if st != 0:
        raise DQError(st, "dq_bench_fp4_mfma_rate")
    return float(out.value)


def solve_outputs(W, fmt: str, group: int, T: int) -> Dict[str, object]:
    """Output tensors for solve_async on W: codes, scales, a, b, mse (T + 1), g."""
    torch = _torch()
    rows, cols = W.shape
    dev = W.device
    codes, scales = _outputs(W, fmt, group)
    return {"codes": codes, "scales": scales,
            "a": torch.empty(rows, dtype=torch.float32, device=dev),
            "b": torch.empty(cols, dtype=torch.float32, device=dev),
            "mse": torch.empty(T + 1, dtype=torch.float64, device=dev),
            "g": torch.zeros(1, dtype=torch.float32, device=dev)}


def solve_async(W, fmt: str, group: int, T: int, out, status, a0=None, b0=None, g0: float = 0.0,
                two_sweep: bool = False, per_pass_g: bool = False, workspace=None,
                stream=None) -> None:
    """dq_solve_async into ``out`` (from solve_outputs): enqueued on the stream, no wait;
    device errors are OR-ed into ``status`` (an int32 CUDA tensor the caller clears)."""
    dt = _check_w(W)
    rows, cols = W.shape
    if out["mse"].numel() != T + 1:
        raise ValueError("out was made for another T")
    a0 = _vec(a0, rows, W.device)
    b0 = _vec(b0, cols, W.device)
    flags = (SOLVE_TWO_SWEEP if two_sweep else 0) | (SOLVE_PER_PASS_G if per_pass_g else 0)
    init = _Init(_ptr(a0), _ptr(b0), float(g0), flags)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().dq_solve_async(W.data_ptr(), DTYPE[dt], rows, cols, FMT[fmt], group, T,
                              ctypes.byref(init), out["codes"].data_ptr(),
                              out["scales"].data_ptr(), out["g"].data_ptr(), out["a"].data_ptr(),
                              out["b"].data_ptr(), out["mse"].data_ptr(), status.data_ptr(),
                              ws_ptr, ws_bytes, _stream(stream))
    if st != 0:
        raise DQError(st, "dq_solve_async")


NOALLOC_SCRATCH_BYTES = 64 << 20  # DQ_NOALLOC_SCRATCH_BYTES


def solve_async_noalloc(W, fmt: str, group: int, T: int, out, status, a0=None, b0=None,
                        g0: float = 0.0, two_sweep: bool = False, per_pass_g: bool = False,
                        stream=None) -> None:
    """dq_solve_async_noalloc into ``out`` (from solve_outputs): as solve_async, with the
    library's per-device scratch as the workspace (no allocation on any path; calls on one GPU
    must not overlap)."""
    dt = _check_w(W)
    rows, cols = W.shape
    if out["mse"].numel() != T + 1:
        raise ValueError("out was made for another T")
    a0 = _vec(a0, rows, W.device)
    b0 = _vec(b0, cols, W.device)
    flags = (SOLVE_TWO_SWEEP if two_sweep else 0) | (SOLVE_PER_PASS_G if per_pass_g else 0)
    init = _Init(_ptr(a0), _ptr(b0), float(g0), flags)
    st = lib().dq_solve_async_noalloc(W.data_ptr(), DTYPE[dt], rows, cols, FMT[fmt], group, T,
                                      ctypes.byref(init), out["codes"].data_ptr(),
                                      out["scales"].data_ptr(), out["g"].data_ptr(),
                                      out["a"].data_ptr(), out["b"].data_ptr(),
                                      out["mse"].data_ptr(), status.data_ptr(), _stream(stream))
    if st != 0:
        raise DQError(st, "dq_solve_async_noalloc")


def quantize(W, fmt: str, group: int, a=None, b=None, g: float = 0.0, workspace=None,
             stream=None) -> Dict[str, object]:
    """dq_quantize: one pass of Q on X(a, b). ``g`` > 0 fixes NVFP4's tensor scale."""
    torch = _torch()
    dt = _check_w(W)
    rows, cols = W.shape
    dev = W.device
    codes, scales = _outputs(W, fmt, group)
    gbuf = torch.full((1,), float(g), dtype=torch.float32, device=dev)
    a = _vec(a, rows, dev)
    b = _vec(b, cols, dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().dq_quantize(W.data_ptr(), DTYPE[dt], rows, cols, FMT[fmt], group, _ptr(a),
                           _ptr(b), gbuf.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                           ws_ptr, ws_bytes, _stream(stream))
    if st != 0:
        raise DQError(st, "dq_quantize")
    return {"codes": codes, "scales": scales, "g": gbuf}


def act_workspace_bytes(tokens: int, cols: int, fmt: str, group: int) -> int:
    return int(lib().dq_act_workspace_bytes(int(tokens), int(cols), FMT[fmt], int(group)))


def quantize_act(X, fmt: str, group: int, b=None, g: float = 0.0, workspace=None,
                 stream=None) -> Dict[str, object]:
    """dq_quantize_act: Q of x = fl32(X * b) per token row (X: tokens x cols, CUDA float32 /
    bfloat16), groups of ``group`` channels. ``g`` > 0 fixes NVFP4's tensor scale, else it is
    computed from X. Returns device tensors codes, scales and g (float32[1])."""
    torch = _torch()
    dt = _check_w(X)
    tokens, cols = X.shape
    dev = X.device
    codes, scales = _outputs(X, fmt, group)
    gbuf = torch.zeros(1, dtype=torch.float32, device=dev)
    b = _vec(b, cols, dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().dq_quantize_act(X.data_ptr(), DTYPE[dt], tokens, cols, FMT[fmt], group, _ptr(b),
                               float(g), gbuf.data_ptr(), codes.data_ptr(), scales.data_ptr(),
                               ws_ptr, ws_bytes, _stream(stream))
    if st != 0:
        raise DQError(st, "dq_quantize_act")
    return {"codes": codes, "scales": scales, "g": gbuf}


def quantize_act_async(X, fmt: str, group: int, codes, scales, status, b=None, g: float = 0.0,
                       gout=None, workspace=None, stream=None) -> None:
    """dq_quantize_act_async into caller-allocated outputs (codes, scales as quantize_act
    returns them, ``status`` an int32 device tensor that collects error bits); no wait."""
    dt = _check_w(X)
    tokens, cols = X.shape
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().dq_quantize_act_async(X.data_ptr(), DTYPE[dt], tokens, cols, FMT[fmt], group,
                                     _ptr(b), float(g), _ptr(gout), codes.data_ptr(),
                                     scales.data_ptr(), status.data_ptr(), ws_ptr, ws_bytes,
                                     _stream(stream))
    if st != 0:
        raise DQError(st, "dq_quantize_act_async")


def gemm_mx(act_codes, act_scales, w_codes, w_scales, a=None, out_dtype: str = "bf16", y=None,
            stream=None):
    """dq_gemm_mx: Y = (xhat Qhat^T) D_a from MXFP4 activation codes / E8M0 scales (tokens x
    K/2, tokens x K/32 uint8, as quantize_act returns them) and weight codes / scales (out x
    K/2, out x K/32, as solve returns them) on the MX-scaled FP4 matrix cores. Returns Y
    (tokens x out, bfloat16 or float32), into ``y`` when given."""
    torch = _torch()
    tokens, out = act_codes.shape[0], w_codes.shape[0]
    K = act_codes.shape[1] * 2
    for t, shape in ((act_codes, (tokens, K // 2)), (act_scales, (tokens, K // 32)),
                     (w_codes, (out, K // 2)), (w_scales, (out, K // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"expected a contiguous CUDA uint8 tensor of shape {shape}")
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    if y is None:
        y = torch.empty((tokens, out), dtype=dt, device=act_codes.device)
    elif y.dtype != dt or tuple(y.shape) != (tokens, out) or not y.is_contiguous():
        raise ValueError("y must be a contiguous tokens x out tensor of the output dtype")
    if a is not None and (a.dtype != torch.float32 or a.numel() != out or not a.is_contiguous()):
        raise ValueError("a must be a contiguous float32 vector of the output channels")
    st = lib().dq_gemm_mx(act_codes.data_ptr(), act_scales.data_ptr(), tokens, K,
                          w_codes.data_ptr(), w_scales.data_ptr(), _ptr(a), out,
                          DTYPE[out_dtype], y.data_ptr(), _stream(stream))
    if st != 0:
        raise DQError(st, "dq_gemm_mx")
    return y


def gemm_pack_weights(w_codes, w_scales, stream=None) -> Dict[str, object]:
    """dq_gemm_pack_weights: the MXFP4 weight codes / E8M0 scales (out x K/2, out x K/32 uint8,
    as solve returns them) laid out for gemm_mx_packed. Returns {"codes", "scales", "out",
    "K"} (device uint8 tensors)."""
    torch = _torch()
    out, K = w_codes.shape[0], w_codes.shape[1] * 2
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib().dq_gemm_pack_bytes(out, K, ctypes.byref(cb), ctypes.byref(sb))
    if st != 0:
        raise DQError(st, "dq_gemm_pack_bytes")
    for t, shape in ((w_codes, (out, K // 2)), (w_scales, (out, K // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"expected a contiguous CUDA uint8 tensor of shape {shape}")
    codes = torch.empty(cb.value, dtype=torch.uint8, device=w_codes.device)
    scales = torch.empty(sb.value, dtype=torch.uint8, device=w_codes.device)
    st = lib().dq_gemm_pack_weights(w_codes.data_ptr(), w_scales.data_ptr(), out, K,
                                    codes.data_ptr(), scales.data_ptr(), _stream(stream))
    if st != 0:
        raise DQError(st, "dq_gemm_pack_weights")
    return {"codes": codes, "scales": scales, "out": out, "K": K}


def gemm_mx_packed(act_codes, act_scales, packed, a=None, out_dtype: str = "bf16", y=None,
                   stream=None):
    """dq_gemm_mx_packed: gemm_mx with weights from gemm_pack_weights."""
    torch = _torch()
    tokens, K, out = act_codes.shape[0], act_codes.shape[1] * 2, packed["out"]
    if K != packed["K"]:
        raise ValueError("activations and packed weights disagree on K")
    for t, shape in ((act_codes, (tokens, K // 2)), (act_scales, (tokens, K // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"expected a contiguous CUDA uint8 tensor of shape {shape}")
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    if y is None:
        y = torch.empty((tokens, out), dtype=dt, device=act_codes.device)
    elif y.dtype != dt or tuple(y.shape) != (tokens, out) or not y.is_contiguous():
        raise ValueError("y must be a contiguous tokens x out tensor of the output dtype")
    if a is not None and (a.dtype != torch.float32 or a.numel() != out or not a.is_contiguous()):
        raise ValueError("a must be a contiguous float32 vector of the output channels")
    st = lib().dq_gemm_mx_packed(act_codes.data_ptr(), act_scales.data_ptr(), tokens, K,
                                 packed["codes"].data_ptr(), packed["scales"].data_ptr(), _ptr(a),
                                 out, DTYPE[out_dtype], y.data_ptr(), _stream(stream))
    if st != 0:
        raise DQError(st, "dq_gemm_mx_packed")
    return y


class _BatchItem(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("a0", ctypes.c_void_p), ("b0", ctypes.c_void_p), ("g0", ctypes.c_float),
                ("codes", ctypes.c_void_p), ("inner_scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("mse", ctypes.c_void_p)]


def _batch_lib():
    L = lib()
    if not getattr(L, "_batch_ready", False):
        P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.dq_batch_workspace_bytes.argtypes = [I, ctypes.POINTER(_BatchItem), I, I]
        L.dq_batch_workspace_bytes.restype = SZ
        L.dq_solve_batch.argtypes = [I, ctypes.POINTER(_BatchItem), I, I, I, I, ctypes.c_uint, P,
                                     P, SZ, P]
        L.dq_solve_batch.restype = I
        L._batch_ready = True
    return L


def solve_batch(Ws, fmt: str, group: int, T: int, per_pass_g: bool = False, workspace=None,
                stream=None):
    """dq_solve_batch on a list of bf16 CUDA matrices (one format and group): every matrix
    solved as dq.solve would solve it, with the per-iteration passes of up to 16 matrices
    sharing each launch. Returns one dict per matrix, as solve() does, with its status."""
    torch = _torch()
    n = len(Ws)
    items = (_BatchItem * n)()
    outs = []
    for k, W in enumerate(Ws):
        if _check_w(W) != "bf16":
            raise ValueError("solve_batch takes bf16 weights")
        rows, cols = W.shape
        codes, scales = _outputs(W, fmt, group)
        o = {"codes": codes, "scales": scales,
             "a": torch.empty(rows, dtype=torch.float32, device=W.device),
             "b": torch.empty(cols, dtype=torch.float32, device=W.device),
             "mse": torch.empty(T + 1, dtype=torch.float64, device=W.device),
             "g": torch.zeros(1, dtype=torch.float32, device=W.device)}
        items[k] = _BatchItem(W.data_ptr(), rows, cols, None, None, 0.0, codes.data_ptr(),
                              scales.data_ptr(), o["g"].data_ptr(), o["a"].data_ptr(),
                              o["b"].data_ptr(), o["mse"].data_ptr())
        outs.append(o)
    L = _batch_lib()
    status = (ctypes.c_int * n)()
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = L.dq_solve_batch(n, items, DTYPE["bf16"], FMT[fmt], group, T,
                          SOLVE_PER_PASS_G if per_pass_g else 0, ctypes.cast(status, ctypes.c_void_p),
                          ws_ptr, ws_bytes, _stream(stream))
    for k in range(n):
        outs[k]["status"] = int(status[k])
    if st != 0:
        raise DQError(st, "dq_solve_batch")
    return outs


def batch_workspace_bytes(shapes, fmt: str, group: int) -> int:
    n = len(shapes)
    items = (_BatchItem * n)()
    for k, (rows, cols) in enumerate(shapes):
        items[k] = _BatchItem(None, rows, cols, None, None, 0.0, None, None, None, None, None, None)
    return int(_batch_lib().dq_batch_workspace_bytes(n, items, FMT[fmt], group))

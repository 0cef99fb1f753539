"""Helpers that move seeded inputs to the GPU and compare the HIP path with the oracle.

The parity bar (DualQuant solver contract): a single Q pass is bit-identical (codes, inner
scales, tensor scale); after T iterations the final mse is within 1e-4 relative, at most
1e-5 of the codes differ, and a, b agree to 1e-4 relative (read as a per-vector relative
l2 error, every differing entry exactly one representable step away).
"""
from __future__ import annotations

import numpy as np

import fmt_brute as fb


def to_device(w_np: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w_np).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w_np)).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def scales_np(gpu_scales, fmt: str) -> np.ndarray:
    s = host(gpu_scales)
    return s.view(np.uint16) if fmt == "int4_bf16" else s


def one_step_apart(fmt: str, x: np.ndarray, y: np.ndarray) -> bool:
    """Whether every pair (x_k, y_k) with x_k != y_k are neighbours in the scale set."""
    for u, v in zip(x.tolist(), y.tolist()):
        if u == v:
            continue
        lo, hi = min(u, v), max(u, v)
        mid = 0.5 * (lo + hi)
        # no representable value strictly between them, checked through the projection
        if fb.project(fmt, mid) not in (lo, hi):
            return False
    return True


def compare_solve(gpu: dict, ref: dict, fmt: str, rows: int, cols: int) -> dict:
    a_g, b_g = host(gpu["a"]), host(gpu["b"])
    codes_g = host(gpu["codes"])
    mse_g = host(gpu["mse"])
    qg = fb.unpack_codes(codes_g, fmt)
    qr = fb.unpack_codes(ref["codes"], fmt)
    rel = lambda x, y: float(np.linalg.norm(x.astype(np.float64) - y) / max(np.linalg.norm(y), 1e-300))
    res = {
        "a_rel_l2": rel(a_g, ref["a"]),
        "b_rel_l2": rel(b_g, ref["b"]),
        "a_flips": int((a_g != ref["a"]).sum()),
        "b_flips": int((b_g != ref["b"]).sum()),
        "a_max_rel": float(np.max(np.abs(a_g.astype(np.float64) - ref["a"]) / ref["a"])),
        "b_max_rel": float(np.max(np.abs(b_g.astype(np.float64) - ref["b"]) / ref["b"])),
        "code_diffs": int((qg != qr).sum()),
        "code_budget": 1e-5 * rows * cols,
        "mse_rel": np.abs(mse_g - ref["mse"]) / np.maximum(ref["mse"], 1e-300),
        "scales_equal": bool(np.array_equal(scales_np(gpu["scales"], fmt), ref["scales"])),
        "steps_ok": one_step_apart(fmt, a_g, ref["a"]) and one_step_apart(fmt, b_g, ref["b"]),
    }
    return res


def assert_parity(res: dict, exact: bool = False, name: str = "") -> None:
    msg = f"{name}: {res}"
    assert res["mse_rel"][-1] <= 1e-4, msg
    assert res["code_diffs"] <= res["code_budget"], msg
    assert res["a_rel_l2"] <= 1e-4 and res["b_rel_l2"] <= 1e-4, msg
    assert res["steps_ok"], msg
    if exact:
        assert res["a_flips"] == 0 and res["b_flips"] == 0 and res["code_diffs"] == 0, msg
        assert res["scales_equal"], msg
        # every per-row error is a sum of nonnegative terms: fp32 over at most 16 exact
        # squares per lane (relative error <= 15 u < 1e-6), fp64 above
        assert np.all(res["mse_rel"] <= 1e-6), msg

"""Format decoders and brute-force rounding for the tests.

Written from the bit layouts of the formats (E2M1, E4M3FN, E8M0, bf16) and from
"nearest value, ties to even mantissa" by enumeration, independently of the
oracle's C code and of the HIP library. The tests use these to pin the oracle
and to decode what either side returns.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Tuple

import numpy as np
import torch

# ------------------------------------------------------------------ E2M1 (FP4)
# 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal.


def e2m1_decode(nib: int) -> float:
    sign = (nib >> 3) & 1
    e = (nib >> 1) & 3
    mnt = nib & 1
    mag = mnt * 0.5 if e == 0 else (1.0 + mnt / 2.0) * 2.0 ** (e - 1)
    return -mag if sign else mag


E2M1_TABLE = np.array([e2m1_decode(c) for c in range(16)], np.float64)
# distinct values with their mantissa bit (for tie-breaking); +0 only
_E2M1_CANDS = [(E2M1_TABLE[c], c & 1) for c in range(16) if c != 8]
_E2M1_VALS = np.array([v for v, _ in _E2M1_CANDS])
_E2M1_MANT = np.array([m for _, m in _E2M1_CANDS])


def e2m1_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value for each entry, ties to the even mantissa bit."""
    v = np.asarray(v, np.float64)
    d = np.abs(v[..., None] - _E2M1_VALS)  # exact for the grid's neighbours (Sterbenz)
    dmin = d.min(axis=-1, keepdims=True)
    at_min = d == dmin
    # among tied candidates keep the even-mantissa one
    pick = np.where(at_min.sum(-1, keepdims=True) > 1, at_min & (_E2M1_MANT == 0), at_min)
    return _E2M1_VALS[np.argmax(pick, axis=-1)]


# ------------------------------------------------------------------ E4M3FN
# bias 7, 3 mantissa bits, exponent 0 subnormal (m * 2^-9), 0x7F / 0xFF are NaN, max 448.


def e4m3_decode(code: int) -> float:
    code &= 0x7F
    e = (code >> 3) & 15
    m = code & 7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_POS_CODES = np.arange(0, 0x7F)  # 0x00 .. 0x7E, non-negative finite
E4M3_POS_VALS = np.array([e4m3_decode(c) for c in E4M3_POS_CODES], np.float64)


def _nearest_in(v: float, vals: np.ndarray, codes: np.ndarray) -> Tuple[float, int]:
    fv = Fraction(v)
    best = None
    for val, code in zip(vals, codes):
        dist = abs(fv - Fraction(float(val)))
        key = (dist, int(code) & 1)  # tie -> even mantissa bit (code LSB)
        if best is None or key < best[0]:
            best = (key, float(val), int(code))
    return best[1], best[2]


def e4m3_nearest_sat(v: float) -> float:
    """Nearest non-negative finite E4M3FN value (which saturates at 448)."""
    return _nearest_in(v, E4M3_POS_VALS, E4M3_POS_CODES)[0]


def e4m3_code_of(val: float) -> int:
    hits = np.nonzero(E4M3_POS_VALS == val)[0]
    assert len(hits) == 1, val
    return int(E4M3_POS_CODES[hits[0]])


# ------------------------------------------------------------------ bf16


def bf16_decode(h) -> np.ndarray:
    h = np.asarray(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def bf16_nearest(v: float) -> Tuple[float, int]:
    """Nearest bf16 value to a finite double v >= 0 by enumeration, ties to even."""
    h0 = int(np.array([v], np.float32).view(np.uint32)[0] >> 16)
    cands = [h for h in range(max(0, h0 - 2), min(0x7F7F, h0 + 2) + 1)]
    vals = bf16_decode(np.array(cands, np.uint16)).astype(np.float64)
    return _nearest_in(v, vals, np.array(cands))


def torch_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (torch's round-to-nearest-even conversion) -> float64."""
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ------------------------------------------------------------------ projections (brute force)
BF16_MIN_NORMAL = 2.0 ** -126
BF16_MAX = float(bf16_decode(np.array([0x7F7F], np.uint16))[0])


def project_bf16(v: float) -> float:
    if v <= BF16_MIN_NORMAL:
        return BF16_MIN_NORMAL
    if v >= BF16_MAX:
        return BF16_MAX
    return bf16_nearest(v)[0]


def project_e8m0(v: float) -> float:
    """Nearest power of two 2^k, k in [-126, 126]; an exact midpoint goes up."""
    fv = Fraction(v)
    best = None
    for k in range(-126, 127):
        p = Fraction(2) ** k
        key = (abs(fv - p), -k)  # tie -> larger k
        if best is None or key < best[0]:
            best = (key, k)
    return 2.0 ** best[1]


def project_e4m3(v: float) -> float:
    """Nearest positive E4M3FN value (0 excluded), ties to even mantissa."""
    return _nearest_in(v, E4M3_POS_VALS[1:], E4M3_POS_CODES[1:])[0]


def project(fmt: str, v: float) -> float:
    return {"int4_bf16": project_bf16, "mxint4": project_e8m0, "mxfp4": project_e8m0,
            "nvfp4": project_e4m3}[fmt](v)


def representable(fmt: str, x: float) -> bool:
    if fmt == "int4_bf16":
        f = np.float32(x)
        return (int(np.array([f]).view(np.uint32)[0]) & 0xFFFF) == 0 and \
            BF16_MIN_NORMAL <= x <= BF16_MAX
    if fmt in ("mxint4", "mxfp4"):
        m, e = np.frexp(x)
        return m == 0.5 and -126 <= e - 1 <= 126
    return bool(np.any(E4M3_POS_VALS[1:] == x))


# ------------------------------------------------------------------ packed outputs


def unpack_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Packed nibbles (column 2k low, 2k+1 high) -> code values (float64)."""
    codes = np.asarray(codes, np.uint8)
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    if fmt in ("int4_bf16", "mxint4"):
        return np.where(nib >= 8, nib.astype(np.int16) - 16, nib).astype(np.float64)
    return E2M1_TABLE[nib]


def decode_scales(scales: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "int4_bf16":
        return bf16_decode(scales).astype(np.float64)
    if fmt in ("mxint4", "mxfp4"):
        return np.ldexp(1.0, scales.astype(np.int64) - 127)
    lut = np.array([e4m3_decode(c) for c in range(256)])
    return lut[scales]


def divisors(scales: np.ndarray, fmt: str, g: float) -> np.ndarray:
    """Per-group divisor d: the scale itself, or fl32(s * g) for NVFP4."""
    s = decode_scales(scales, fmt)
    if fmt == "nvfp4":
        return (s.astype(np.float32) * np.float32(g)).astype(np.float64)
    return s


def dequant(codes: np.ndarray, scales: np.ndarray, fmt: str, group: int, g: float) -> np.ndarray:
    """Qhat = code * d, rows x cols, float64."""
    q = unpack_codes(codes, fmt)
    d = divisors(scales, fmt, g)
    return q * np.repeat(d, group, axis=1)


def scaled_tile(W32: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """X = fl32(fl32(W * fl32(1/b)) * fl32(1/a)) with numpy float32 (IEEE) arithmetic."""
    ra = (np.float32(1.0) / a.astype(np.float32)).astype(np.float32)
    rb = (np.float32(1.0) / b.astype(np.float32)).astype(np.float32)
    y = (W32 * rb[None, :]).astype(np.float32)
    return (y * ra[:, None]).astype(np.float32)

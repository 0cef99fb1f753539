"""Exhaustive GPU check of gfx950's FP4 conversion as the kernels use it, against exact E2M1
rounding (tests/fmt_brute.py's grid, nearest value, ties to the even index, saturating at 6;
the MXFP4 and NVFP4 elements of the block formats in the yiqijian article, "适配 MXFP4 与
NVFP4 块结构").

- v_cvt_scalef32_pk_fp4_f32 with every power-of-two scale the MX kernels pass it (2^-100 ..
  2^29: the activation quantizer uses it for 2^-100 .. 2^20, the single-sweep solver pass for
  group scales 2^-34 .. 2^29), on every non-negative finite fp32 input and its negation, at
  every byte position;
- the NVFP4 fp32 codes (nv_pack8_fast: an odd-rounded quotient, then that conversion with
  scale 1), with and without its clamp, for E4M3 scales times several tensor scales;
- v_cvt_scalef32_pk_f32_fp4, the decode the single-sweep pass forms code * scale with, for
  every byte and position;
- that both read only the exponent field of their fp32 scale: the single-sweep MXFP4 pass
  passes the group maximum's own bit pattern with two taken off its exponent (a saturating
  subtract, so an all-zero group passes exponent field 0), mantissa bits and all.

How one scan covers every input: the probe (tests/fp4_scan.hip) records the bit patterns
where the code of x changes as x rises. Exact E2M1 rounding of x / d is a non-decreasing
step function of x >= 0, and so is what the probe saw between its recorded points (constant).
The test checks the code at 0, at the last input, and on both sides of every recorded
transition against exact rounding; by monotonicity the two functions then agree on every
input in between."""
import ctypes
from fractions import Fraction

import numpy as np
import pytest

import fmt_brute as fb
import probes

pytestmark = pytest.mark.gpu

CAP = 64
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]
MAX_FINITE = 0x7F7FFFFF


@pytest.fixture(scope="module")
def P():
    import torch

    assert torch.cuda.is_available()
    return probes.lib()


def _val(u):
    return float(np.array([u], np.uint32).view(np.float32)[0])


def _e2m1_index(q: Fraction) -> int:
    """Index 0..7 of the E2M1 value nearest to q >= 0 (ties to the even index, saturating)."""
    best = min(range(8), key=lambda k: (abs(q - GRID[k]), k & 1))
    return best


def _scan(P, mode, p, u_last):
    import torch

    res = torch.zeros(4 + 3 * CAP, dtype=torch.int32, device="cuda")
    st = P.fp4_scan(mode, float(p), u_last, ctypes.c_void_p(res.data_ptr()), CAP, None)
    assert st == 0, st
    torch.cuda.synchronize()
    r = res.cpu().numpy().view(np.uint32)
    return r


def _check_scan(r, ref_index, u_last, what):
    count, neg_bad, first_bad, pos_bad = (int(v) for v in r[:4])
    assert pos_bad == 0, (what, "byte positions disagree", pos_bad)
    assert neg_bad == 0, (what, "sign of -x", neg_bad, hex(first_bad))
    assert count <= CAP, (what, "more transitions than E2M1 has", count)
    trans = sorted((int(r[4 + 3 * k]), int(r[5 + 3 * k]), int(r[6 + 3 * k])) for k in range(count))
    # the code at 0, on both sides of every transition, and at the last input
    points = [(0, None)]
    for u, c0, c1 in trans:
        assert c1 > c0, (what, "codes of a rising x fell", u, c0, c1)
        points += [(u, c0), (u + 1, c1)]
    last_code = trans[-1][2] if trans else None
    points.append((u_last, last_code))
    start_code = trans[0][1] if trans else last_code
    for u, code in points:
        want = ref_index(_val(u))
        got = start_code if code is None else code
        assert got == want, (what, hex(u), _val(u), got, want)
    return count


MX_SCALE_EXPONENTS = list(range(-100, 30))


def test_mx_conversion_every_input_every_scale(P):
    seen = 0
    for k in MX_SCALE_EXPONENTS:
        p = 2.0 ** k
        r = _scan(P, 0, p, MAX_FINITE)
        ref = lambda x, p=p: _e2m1_index(Fraction(x) / Fraction(p))
        n = _check_scan(r, ref, MAX_FINITE, f"scale 2^{k}")
        assert n == 7, (k, n)  # 0 -> 0.5 -> ... -> 6: seven transitions, all inside the range
        seen += n
    print(f"[fp4] {len(MX_SCALE_EXPONENTS)} scales x {MAX_FINITE + 1} inputs: {seen} transitions", flush=True)


def _nv_divisors():
    s_vals = [float(v) for v in fb.E4M3_POS_VALS[1:]]
    out = []
    for g in (1.0, 3.0 / 256.0, 0.0071, 2.0 ** -80 * 1.7, 2.0 ** 60 * 1.3):
        g32 = np.float32(g)
        for s in s_vals[::5] + [s_vals[-1]]:
            d = float(np.float32(np.float64(s) * np.float64(g32)))
            if 2.0 ** -100 <= d <= 2.0 ** 100:
                out.append(d)
    return sorted(set(out))


def _last_below(limit):
    """Largest non-negative fp32 bit pattern whose value is below limit."""
    v = np.float32(limit)
    if float(v) >= limit:
        v = np.nextafter(v, np.float32(0))
    return int(np.array([v], np.float32).view(np.uint32)[0])


def test_nvfp4_fp32_codes_every_input(P):
    divs = _nv_divisors()
    assert len(divs) > 60
    for d in divs:
        ref = lambda x, d=d: _e2m1_index(Fraction(x) / Fraction(d))
        r = _scan(P, 1, d, MAX_FINITE)  # with the clamp at 8 d: every input
        assert _check_scan(r, ref, MAX_FINITE, f"clamped d={d!r}") == 7
        u7 = _last_below(7.0 * d)  # without it: inputs below 7 d, as its callers guarantee
        r = _scan(P, 2, d, u7)
        assert _check_scan(r, ref, u7, f"unclamped d={d!r}") == 7
    print(f"[fp4] NVFP4 fp32 codes: {len(divs)} divisors, every input", flush=True)


@pytest.mark.parametrize("k", [-34, -10, -1, 0, 1, 20, 29])
def test_fp4_decode_every_byte(P, k):
    import torch

    p = 2.0 ** k
    out = torch.zeros(2048, dtype=torch.float32, device="cuda")
    assert P.fp4_decode(float(p), ctypes.c_void_p(out.data_ptr()), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(4, 256, 2).astype(np.float64)
    byte = np.arange(256)
    want = np.stack([fb.E2M1_TABLE[byte & 0xF], fb.E2M1_TABLE[byte >> 4]], axis=-1) * p
    for pos in range(4):
        assert np.array_equal(got[pos], want), (k, pos)


# scales as the single-sweep pass forms them: exponent field e, arbitrary mantissa bits
SCALE_MANTISSAS = [0x7FFFFF, 0x400000, 0x2A5A5B]


def _scale_bits(k, m):
    return float(np.array([((k + 127) << 23) | m], np.uint32).view(np.float32)[0])


@pytest.mark.parametrize("k", [-34, -3, 0, 7, 29])
def test_mx_conversion_reads_only_the_scale_exponent(P, k):
    import torch

    for m in SCALE_MANTISSAS:
        p = _scale_bits(k, m)
        r = _scan(P, 0, p, MAX_FINITE)
        ref = lambda x: _e2m1_index(Fraction(x) / Fraction(2) ** k)
        assert _check_scan(r, ref, MAX_FINITE, f"scale 2^{k} with mantissa {m:#x}") == 7
        out = torch.zeros(2048, dtype=torch.float32, device="cuda")
        assert P.fp4_decode(p, ctypes.c_void_p(out.data_ptr()), None) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(4, 256, 2).astype(np.float64)
        byte = np.arange(256)
        want = np.stack([fb.E2M1_TABLE[byte & 0xF], fb.E2M1_TABLE[byte >> 4]], axis=-1) * 2.0 ** k
        for pos in range(4):
            assert np.array_equal(got[pos], want), (k, hex(m), pos)


def test_all_zero_group_with_exponent_field_zero(P):
    # an all-zero group's scale is 0 (or, below 2^-125, a value with exponent field 0): its
    # codes are 0 (+0 and -0 inputs alike, magnitude 0) and code 0 decodes to 0
    import torch

    x = torch.tensor([0.0, -0.0, -0.0, 0.0, 0.0, 0.0], dtype=torch.float32, device="cuda")
    out = torch.full((3,), 0xFF, dtype=torch.int32, device="cuda")
    for p in (0.0, _scale_bits(-127, 0x7FFFFF), _scale_bits(-127, 0x000001)):
        assert P.fp4_encode(p, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), 3,
                            None) == 0
        dec = torch.ones(2048, dtype=torch.float32, device="cuda")
        assert P.fp4_decode(p, ctypes.c_void_p(dec.data_ptr()), None) == 0
        torch.cuda.synchronize()
        codes = out.cpu().numpy().astype(np.uint32)
        assert np.all((codes & 0x77) == 0), (p, codes)
        d = dec.cpu().numpy().reshape(4, 256, 2)
        assert np.all(d[:, 0, :] == 0.0), p  # byte 0 at every position

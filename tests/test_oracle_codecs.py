"""Pins for the oracle's scalar pieces: rounding to E2M1 / E4M3 / bf16 and the
projections Pi_F of the outer inverse scales (daiwk notes, "核心公式": the
projection maps the closed-form inverse scale to the format's representable set;
"本地复现": BF16 scales, E8M0 exponent in [-126, 126]; news article's block-format
paragraph: E2M1 elements, E8M0 / E4M3 block scales).

Every expected value comes from enumerating the format's encodings (tests/fmt_brute.py)
or from torch's own float32 -> bfloat16 / float8_e4m3fn conversions.
"""
import math

import numpy as np
import pytest
import torch

import fmt_brute as fb


def _e2m1_test_values():
    grid = sorted(set(abs(float(v)) for v in fb.E2M1_TABLE))
    mids = [(x + y) / 2 for x, y in zip(grid, grid[1:])]
    vals = set(grid + mids + [7.0, 8.0, 100.0, 1e-30, 5e-324])
    for v in list(vals):
        vals.add(math.nextafter(v, math.inf))
        vals.add(math.nextafter(v, -math.inf))
    rng = np.random.default_rng(5)
    vals.update(rng.uniform(0, 8, 2000).tolist())
    vals = [v for v in vals if v >= 0]
    return sorted(vals + [-v for v in vals])


def test_e2m1_round_matches_enumeration(oracle_lib):
    vals = _e2m1_test_values()
    got = np.array([oracle_lib.e2m1_round(v) for v in vals])
    want = fb.e2m1_nearest(np.array(vals))
    assert np.array_equal(got, want)
    # no negative zero comes back
    assert not any(math.copysign(1.0, g) < 0 for g in got if g == 0)


def test_e2m1_ties_go_to_even_index(oracle_lib):
    # the pages' E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}: every midpoint resolves to the
    # neighbour with mantissa bit 0
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, w in expect.items():
        assert oracle_lib.e2m1_round(v) == w
        assert oracle_lib.e2m1_round(-v) == (-w if w else 0.0)


def _e4m3_test_values():
    vals = set(fb.E4M3_POS_VALS.tolist())
    pos = sorted(vals)
    vals.update(((x + y) / 2 for x, y in zip(pos, pos[1:])))
    vals.update([456.0, 464.0, 465.0, 1e6, 2.0 ** -10, 3 * 2.0 ** -11, 1e-45])
    for v in list(vals):
        vals.add(math.nextafter(v, math.inf))
        if v > 0:
            vals.add(math.nextafter(v, 0))
    rng = np.random.default_rng(7)
    vals.update(np.exp(rng.uniform(math.log(2.0 ** -12), math.log(600.0), 1500)).tolist())
    return sorted(vals)


def test_e4m3_rne_sat_matches_enumeration(oracle_lib):
    for v in _e4m3_test_values():
        assert oracle_lib.e4m3_rne_sat(v) == fb.e4m3_nearest_sat(v), v


def test_e4m3_matches_torch_float8(oracle_lib):
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even; compare where
    # it is defined (|v| <= 448; it does not saturate above)
    rng = np.random.default_rng(8)
    x = np.concatenate([np.exp(rng.uniform(-12, 6.1, 5000)), fb.E4M3_POS_VALS]).astype(np.float32)
    x = x[x <= 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_lib.e4m3_rne_sat(float(v)) for v in x])
    assert np.array_equal(got, t)


def test_bf16_rne_matches_torch_on_all_upper_halves(oracle_lib):
    # every bf16 upper half with the low halves that decide rounding: exact, just
    # below / at / above the tie, and the extremes
    hi = np.arange(0, 0x7F80, dtype=np.uint32)  # non-negative finite upper halves
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4321], np.uint32)
    bits = (hi[:, None] << 16 | lows[None, :]).reshape(-1)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (x < fb.BF16_MAX)]
    want = fb.torch_bf16(x)
    f = oracle_lib.lib().dq_ref_bf16_rne
    got = np.fromiter((f(float(v)) for v in x), np.float64, count=len(x))
    assert np.array_equal(got, want)


def test_bf16_rne_matches_enumeration_on_doubles(oracle_lib):
    rng = np.random.default_rng(9)
    vals = np.exp(rng.uniform(math.log(1e-41), math.log(1e30), 600))
    for v in vals:
        assert oracle_lib.bf16_rne(float(v)) == fb.bf16_nearest(float(v))[0]


@pytest.mark.parametrize("fmt", ["int4_bf16", "mxint4", "nvfp4"])
def test_projection_is_nearest_representable(oracle_lib, fmt):
    rng = np.random.default_rng(10)
    vals = list(np.exp(rng.uniform(math.log(1e-3), math.log(1e3), 300)))
    if fmt == "int4_bf16":
        # midpoints between neighbouring bf16 values, exact ties and 1 ulp off
        base = fb.bf16_decode(np.array([0x3F80, 0x3F81, 0x4000, 0x3A55, 0x4A10], np.uint16))
        step = np.ldexp(1.0, np.frexp(base.astype(np.float64))[1] - 8)
        mids = base.astype(np.float64) + step / 2
        vals += list(mids) + [math.nextafter(m, 0) for m in mids] + \
            [math.nextafter(m, math.inf) for m in mids] + [1e-39, 1e-300, 3.5e38, 1e300]
    elif fmt == "mxint4":
        ks = np.arange(-128, 129)
        mids = 1.5 * np.ldexp(1.0, ks)
        vals += list(mids) + [math.nextafter(m, 0) for m in mids] + [1e-300, 1e300]
    else:
        pos = fb.E4M3_POS_VALS[1:]
        mids = (pos[1:] + pos[:-1]) / 2
        vals += list(mids) + [math.nextafter(m, 0) for m in mids] + \
            [math.nextafter(m, math.inf) for m in mids] + [1e-6, 2.0 ** -10, 1000.0, 1e300]
    for v in vals:
        got = oracle_lib.project(fmt, float(v))
        assert got == fb.project(fmt, float(v)), (fmt, v, got)
        assert fb.representable(fmt, got)


def test_e8m0_projection_range_is_pinned_to_pages(oracle_lib):
    # daiwk notes, "本地复现": E8M0 power-of-two scales with exponent in [-126, 126]
    assert oracle_lib.project("mxfp4", 1e-300) == 2.0 ** -126
    assert oracle_lib.project("mxfp4", 1e300) == 2.0 ** 126
    assert oracle_lib.project("mxfp4", 1.5) == 2.0  # midpoint goes up (reading)
    assert oracle_lib.project("mxfp4", math.nextafter(1.5, 0)) == 1.0

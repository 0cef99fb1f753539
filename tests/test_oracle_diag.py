"""Pins for the oracle's diagnostics, which the GPU parity tests rely on.

- The projection margin decides whether a GPU solve must match the oracle exactly (no
  projection decision within 1e-9 of a boundary) or only to the solver contract. It is
  pinned here against the nearest midpoint between neighbouring values of the scale set,
  found by enumerating the set (bf16 around v, every E8M0 power of two, every positive
  E4M3 value) and measured exactly with rationals.
- The change counts (codes and inner scales that differ between consecutive Q passes)
  decide which iterations the conditional-descent pin checks. They are pinned against
  numpy differences of separate Q passes at the intermediate states, which come from
  shorter solves (the state after t iterations is the result of a T = t solve, and the row
  update of iteration t leaves the a of a T = t + 1 solve with the b of a T = t one).
"""
from fractions import Fraction

import numpy as np
import pytest

import fmt_brute as fb
from cases import rand_w

FMTS = ["int4_bf16", "mxint4", "mxfp4", "nvfp4"]


def _scale_set_near(fmt, v):
    """Sorted values of the format's outer scale set around v (the whole set for E8M0 and
    E4M3; for bf16 every value within a few steps of v, plus the range's ends)."""
    if fmt in ("mxint4", "mxfp4"):
        return [Fraction(2) ** k for k in range(-126, 127)]
    if fmt == "nvfp4":
        return sorted(Fraction(float(x)) for x in fb.E4M3_POS_VALS[1:])
    vv = min(max(v, fb.BF16_MIN_NORMAL), fb.BF16_MAX)
    h0 = int(np.array([vv], np.float32).view(np.uint32)[0] >> 16)
    lo, hi = 0x0080, 0x7F7F  # smallest normal and largest finite bf16
    hs = range(max(lo, h0 - 4), min(hi, h0 + 4) + 1)
    return [Fraction(float(x)) for x in fb.bf16_decode(np.array(list(hs), np.uint16))]


def _brute_margin(fmt, v):
    vals = _scale_set_near(fmt, v)
    mids = [(x + y) / 2 for x, y in zip(vals[:-1], vals[1:])]
    fv = Fraction(v)
    return float(min(abs(fv - t) for t in mids) / fv)


def _probe_values(fmt, rng):
    out = list(np.exp(rng.uniform(np.log(1e-6), np.log(1e6), 60)))
    # exact midpoints and values just beside them, the scale-set values themselves
    for _ in range(20):
        x = float(fb.project(fmt, float(np.exp(rng.uniform(np.log(1e-3), np.log(1e3))))))
        nxt = float(fb.project(fmt, x * 1.3)) if fmt == "nvfp4" else None
        if fmt in ("mxint4", "mxfp4"):
            mid = 1.5 * x
        elif fmt == "nvfp4":
            mid = 0.5 * (x + nxt) if nxt != x else x
        else:
            mid = x * (1.0 + 2.0 ** -8)  # between x and its upper neighbour
        out += [x, mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    # around the ends of the scale sets
    if fmt == "int4_bf16":
        out += [2.0 ** -127, 2.0 ** -126, 2.0 ** -126 * 1.004, fb.BF16_MAX * 0.999, 1e39]
    elif fmt == "nvfp4":
        out += [2.0 ** -11, 2.0 ** -9, 1.5 * 2.0 ** -9, 440.0, 448.0, 460.0, 500.0]
    else:
        out += [2.0 ** -127, 2.0 ** -126, 2.0 ** 126, 2.0 ** 127 * 1.4]
    return [float(v) for v in out]


@pytest.mark.parametrize("fmt", FMTS)
def test_proj_margin_is_the_distance_to_the_nearest_decision_point(oracle_lib, fmt):
    rng = np.random.default_rng(list(FMTS).index(fmt) + 41)
    for v in _probe_values(fmt, rng):
        got = oracle_lib.proj_margin(fmt, v)
        want = _brute_margin(fmt, v)
        assert abs(got - want) <= 1e-12 * max(want, 1e-300) or got == want, (fmt, v, got, want)


def _unpacked(out, fmt):
    return fb.unpack_codes(out["codes"], fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_change_counts_match_separate_q_passes(oracle_lib, fmt):
    group = 16 if fmt == "nvfp4" else 32
    W = rand_w(48, 256, seed=73, outliers=6)
    T = 4
    full = oracle_lib.solve(W, "f32", fmt, group, T, diag=True)
    g = full["g"]
    # state after t iterations, t = 0 .. T (a solve of T = t iterations ends there)
    states = [(np.ones(48, np.float32), np.ones(256, np.float32))]
    for t in range(1, T + 1):
        r = oracle_lib.solve(W, "f32", fmt, group, t)
        states.append((r["a"], r["b"]))
    assert np.array_equal(states[T][0], full["a"]) and np.array_equal(states[T][1], full["b"])
    moved = 0
    for t in range(T):
        a_t, b_t = states[t]
        a_next, b_next = states[t + 1]
        qa = oracle_lib.quantize(W, "f32", fmt, group, a_t, b_t, g)      # synced state
        qb = oracle_lib.quantize(W, "f32", fmt, group, a_next, b_t, g)   # after the row update
        qc = oracle_lib.quantize(W, "f32", fmt, group, a_next, b_next, g)  # after the column one
        want = [int((_unpacked(qa, fmt) != _unpacked(qb, fmt)).sum()),
                int((qa["scales"] != qb["scales"]).sum()),
                int((_unpacked(qb, fmt) != _unpacked(qc, fmt)).sum()),
                int((qb["scales"] != qc["scales"]).sum())]
        assert list(full["changes"][t]) == want, (fmt, t, list(full["changes"][t]), want)
        moved += sum(want)
    assert moved > 0  # the counts were not all zero (the pin would then see no index slip)

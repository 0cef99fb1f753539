"""Pins of the oracle's NVFP4 variant with a per-pass tensor scale (dq_ref_solve_pass_g):
g = fl32(max|X| / 2688) of the scaled tile about to be quantized, before every Q pass.

Against independent recomputation: each iteration equals the projected least-squares
updates computed with numpy.linalg.lstsq and brute-force projection, where every Q pass
uses the g of its own tile (the oracle's single Q pass computes that g, pinned by brute force
in test_oracle_solver.py); the final g is recomputed from the final scaled tile in numpy.
Invariants: T = 0 equals the frozen-g solve, a solve resumes exactly from (a, b) alone, and
scaling W by a power of two scales g by it and keeps a, b, codes and inner scales."""
import numpy as np
import pytest

import fmt_brute as fb
from cases import rand_w
from test_oracle_solver import _expected_step, _w32

G = 16


def _final_g(W32, a, b):
    X = fb.scaled_tile(W32, a, b)
    A = np.float32(np.abs(X).max())
    if A == 0:
        return np.float32(1.0)
    return max(np.float32(A / np.float32(2688.0)), np.float32(2.0 ** -126))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_iterations_are_projected_least_squares_with_their_own_g(oracle_lib, dtype):
    W = rand_w(24, 6 * G, seed=41, dtype=dtype, outliers=5)
    W32 = _w32(W, dtype)
    a = np.ones(24, np.float32)
    b = np.ones(6 * G, np.float32)
    for t in range(4):
        a_exp, b_exp = _expected_step(W32, "nvfp4", G, a, b, 0.0, oracle_lib, dtype, W)
        nxt = oracle_lib.solve_pass_g(W, dtype, G, 1, a0=a, b0=b)
        assert np.array_equal(nxt["a"], a_exp), t
        assert np.array_equal(nxt["b"], b_exp), t
        assert np.float32(nxt["g"]) == _final_g(W32, nxt["a"], nxt["b"])
        a, b = nxt["a"], nxt["b"]


def test_zero_iterations_equal_the_frozen_solve(oracle_lib):
    W = rand_w(20, 8 * G, seed=42, outliers=4)
    x = oracle_lib.solve_pass_g(W, "f32", G, 0)
    y = oracle_lib.solve(W, "f32", "nvfp4", G, 0)
    for k in ("codes", "scales", "a", "b", "mse"):
        assert np.array_equal(x[k], y[k]), k
    assert x["g"] == y["g"]


def test_resume_from_the_outer_scales_alone(oracle_lib):
    W = rand_w(30, 8 * G, seed=43, outliers=6)
    full = oracle_lib.solve_pass_g(W, "f32", G, 7)
    first = oracle_lib.solve_pass_g(W, "f32", G, 3)
    rest = oracle_lib.solve_pass_g(W, "f32", G, 4, a0=first["a"], b0=first["b"])
    for k in ("codes", "scales", "a", "b"):
        assert np.array_equal(rest[k], full[k]), k
    assert rest["g"] == full["g"]
    assert np.array_equal(np.concatenate([first["mse"][:3], rest["mse"]]), full["mse"])


def test_power_of_two_equivariance(oracle_lib):
    W = rand_w(30, 8 * G, seed=44, outliers=6)
    base = oracle_lib.solve_pass_g(W, "f32", G, 5)
    for k in (-7, 5):
        sc = oracle_lib.solve_pass_g(W * np.float32(2.0 ** k), "f32", G, 5)
        for key in ("codes", "scales", "a", "b"):
            assert np.array_equal(sc[key], base[key]), (k, key)
        assert sc["g"] == base["g"] * 2.0 ** k
        assert np.allclose(sc["mse"], base["mse"] * 4.0 ** k, rtol=1e-12, atol=0)


def test_differs_from_the_frozen_scale_once_the_tile_moves(oracle_lib):
    # with g frozen at the initial tile the final g is the initial one; per pass it follows
    # the final tile (and the two solves are different readings of the same method). Row 0
    # holds the tile max: one value of 6 units per group and the rest at 4.5 units, which Q
    # rounds down to 4, so the row's least-squares scale is about 1.11 and a_0 becomes 1.125;
    # the tile max then shrinks, and so does the per-pass g.
    W = rand_w(40, 8 * G, seed=45, outliers=0)
    u = np.float32(np.abs(W).max() * 4)
    W[0, :] = np.float32(0.75) * u
    W[0, ::G] = u
    frozen = oracle_lib.solve(W, "f32", "nvfp4", G, 6)
    pp = oracle_lib.solve_pass_g(W, "f32", G, 6)
    assert frozen["g"] == _final_g(W, np.ones(40, np.float32), np.ones(8 * G, np.float32))
    assert pp["a"][0] == np.float32(1.125)
    assert np.float32(pp["g"]) == _final_g(W, pp["a"], pp["b"])
    assert np.float32(pp["g"]) < np.float32(frozen["g"])
    assert not np.array_equal(pp["codes"], frozen["codes"])

"""Pins for the oracle's quantizer Q and its block-coordinate-descent solver.

The method (daiwk notes, "核心公式" eq. 1-2 and the conventions under them; trove
summary, "How it works"): with codes fixed, the row update is the 1-D least-squares
scale of W_i against R_i = (Qhat D_b)_i, projected onto the format's scale set; then
Q is re-run with the synced inner copies; then the column update is the 1-D
least-squares scale of W_:j against S_:j = (D_a Qhat)_:j, projected; then Q again.

Nothing here re-types the oracle's arithmetic. Expected values come from
numpy.linalg.lstsq and exact rational least squares, brute-force enumeration of
representable values and codes, torch / numpy IEEE conversions, and invariants
(idempotence, fixed points, zero slices, equivariance, resume, descent).
"""
from fractions import Fraction

import numpy as np
import pytest

import fmt_brute as fb
from qbrute import check_q_output
from cases import adversarial_w as _adversarial_w
from cases import rand_w as _rand_w

FMTS = ["int4_bf16", "mxint4", "mxfp4", "nvfp4"]
GROUP = {"int4_bf16": 32, "mxint4": 32, "mxfp4": 32, "nvfp4": 16}


def _w32(W, dtype):
    return W if dtype == "f32" else fb.bf16_decode(W)


def _qhat(out, fmt, group):
    return fb.dequant(out["codes"], out["scales"], fmt, group, out["g"])


def _ls_scale(target, basis):
    """argmin_s ||target - s * basis||^2 via numpy.linalg.lstsq (0 for an all-zero basis)."""
    if not np.any(basis):
        return None
    sol = np.linalg.lstsq(basis[:, None], target, rcond=None)[0]
    return float(sol[0])


def _expected_step(W32, fmt, group, a, b, g, oracle_lib, dtype, W):
    """One iteration from (a, b) computed with lstsq + brute-force projection, using the
    oracle's Q only to obtain the codes of each (pinned separately below)."""
    q0 = oracle_lib.quantize(W, dtype, fmt, group, a, b, g)
    R = _qhat(q0, fmt, group) * b[None, :].astype(np.float64)
    a_new = np.empty_like(a)
    for i in range(W32.shape[0]):
        s = _ls_scale(W32[i].astype(np.float64), R[i])
        a_new[i] = 1.0 if s is None else fb.project(fmt, s)
    q1 = oracle_lib.quantize(W, dtype, fmt, group, a_new, b, g)
    S = a_new[:, None].astype(np.float64) * _qhat(q1, fmt, group)
    b_new = np.empty_like(b)
    for j in range(W32.shape[1]):
        s = _ls_scale(W32[:, j].astype(np.float64), S[:, j])
        b_new[j] = 1.0 if s is None else fb.project(fmt, s)
    return a_new, b_new


@pytest.mark.parametrize("fmt", FMTS)
def test_updates_are_projected_least_squares(oracle_lib, fmt):
    group = GROUP[fmt]
    dtype = "bf16" if fmt != "int4_bf16" else "f32"
    W = _rand_w(24, 6 * group, seed=11 + FMTS.index(fmt), dtype=dtype)
    W32 = _w32(W, dtype)
    W32[3, :] = 0  # a zero row -> a = 1
    if dtype == "bf16":
        W[3, :] = 0
    st = oracle_lib.solve(W, dtype, fmt, group, 0)
    a, b, g = st["a"], st["b"], st["g"]
    for t in range(4):
        a_exp, b_exp = _expected_step(W32, fmt, group, a, b, g, oracle_lib, dtype, W)
        nxt = oracle_lib.solve(W, dtype, fmt, group, 1, a0=a, b0=b, g0=g)
        assert np.array_equal(nxt["a"], a_exp), (fmt, t)
        assert np.array_equal(nxt["b"], b_exp), (fmt, t)
        a, b = nxt["a"], nxt["b"]
    assert a[3] == 1.0


def test_row_update_exact_rational(oracle_lib):
    # eq. 2 (left) in exact arithmetic on a tiny INT4/BF16 slice
    W = _rand_w(3, 32, seed=3)
    q0 = oracle_lib.quantize(W, "f32", "int4_bf16", 32)
    Qh = _qhat(q0, "int4_bf16", 32)
    out = oracle_lib.solve(W, "f32", "int4_bf16", 32, 1)
    for i in range(3):
        N = sum(Fraction(float(w)) * Fraction(float(r)) for w, r in zip(W[i], Qh[i]))
        D = sum(Fraction(float(r)) ** 2 for r in Qh[i])
        assert out["a"][i] == fb.project("int4_bf16", float(N / D))


# ------------------------------------------------------------------ Q against brute force

def _check_q_brute(oracle_lib, W32, fmt, group, a, b, g_in, samples=3000, seed=0):
    out = oracle_lib.quantize(W32, "f32", fmt, group, a, b, g_in)
    rows, cols = W32.shape
    A = np.ones(rows, np.float32) if a is None else a
    B = np.ones(cols, np.float32) if b is None else b
    check_q_output(out, fb.scaled_tile(W32, A, B), fmt, group, g_in, samples, seed)
    return out


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("group", [16, 32, 64])
def test_quantizer_matches_brute_force(oracle_lib, fmt, group):
    W = _adversarial_w(fmt, group, 20, seed=group)
    _check_q_brute(oracle_lib, W, fmt, group, None, None, 0.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantizer_with_scales_matches_brute_force(oracle_lib, fmt):
    rng = np.random.default_rng(21)
    group = GROUP[fmt]
    W = _rand_w(16, 4 * group, seed=22)
    a = np.array([fb.project(fmt, v) for v in rng.uniform(0.3, 3, 16)], np.float32)
    b = np.array([fb.project(fmt, v) for v in rng.uniform(0.3, 3, 4 * group)], np.float32)
    _check_q_brute(oracle_lib, W, fmt, group, a, b, 0.0)
    if fmt == "nvfp4":
        _check_q_brute(oracle_lib, W, fmt, group, a, b, 1.7e-5)  # a given tensor scale


def test_scaled_tile_rounds_the_column_scale_first(oracle_lib):
    """Reading 5 fixes the order of the two fp32 roundings of the scaled tile: X =
    fl32(fl32(W * fl32(1/b)) * fl32(1/a)). At the top of the fp32 range the order decides
    whether a value overflows: with W = 2^127, 1/b = 2 and 1/a = 1/4 the column scale first
    gives fl32(2^128) = inf (a range error), the row scale first would give 2^126."""
    from oracle import OracleError

    for fmt in ("int4_bf16", "nvfp4"):  # outer scales that may be any bf16 / E4M3 value
        group = GROUP[fmt]
        W = np.zeros((1, group), np.float32)
        W[0, 0] = np.float32(2.0 ** 127)
        a = np.array([4.0], np.float32)
        b = np.ones(group, np.float32)
        b[0] = 0.5
        with pytest.raises(OracleError) as e:
            oracle_lib.quantize(W, "f32", fmt, group, a, b, 1.0 if fmt == "nvfp4" else 0.0)
        assert e.value.status == 4  # DQR_ERR_RANGE
        # the same magnitudes with the scales swapped stay finite in this order
        out = oracle_lib.quantize(W, "f32", fmt, group, np.array([0.5], np.float32),
                                  np.where(b == 0.5, np.float32(4.0), b), 1.0 if fmt == "nvfp4" else 0.0)
        X = fb.scaled_tile(W, np.array([0.5], np.float32), np.where(b == 0.5, np.float32(4.0), b))
        assert np.isfinite(X).all()
        if fmt == "int4_bf16":  # (NVFP4 with g = 1 saturates its scale at this size)
            check_q_output(out, X, fmt, group, 0.0, samples=group)


def test_int4_scale_floor_for_the_smallest_groups(oracle_lib):
    """Reading 1: INT4_BF16's s = max(bf16(fl32(m/7)), 2^-133). A group whose max is the
    smallest fp32 subnormal has m/7 below half the smallest bf16 subnormal, so bf16 rounding
    gives 0 and the floor gives s = 2^-133 (bits 0x0001); its values quantize to 0."""
    W = np.zeros((2, 16), np.float32)
    W[0, 3] = np.float32(2.0 ** -149)
    W[1, 5] = -np.float32(2.0 ** -140)
    out = oracle_lib.quantize(W, "f32", "int4_bf16", 16)
    assert out["scales"].tolist() == [[0x0001], [0x0001]]  # both below 7 * 2^-134
    assert not out["codes"].any()


# ------------------------------------------------------------------ invariants

def test_zero_slices_take_scale_one(oracle_lib):
    # daiwk notes, "核心公式": an all-zero code slice uses the scale-1 convention
    for fmt in FMTS:
        group = GROUP[fmt]
        W = _rand_w(12, 4 * group, seed=31)
        W[2, :] = 0
        W[:, 5] = 0
        W[7, group:2 * group] = 0
        out = oracle_lib.solve(W, "f32", fmt, group, 3)
        assert out["a"][2] == 1.0
        assert out["b"][5] == 1.0
        s = fb.decode_scales(out["scales"], fmt)
        assert np.all(s[2] == 1.0) and s[7, 1] == 1.0
        q = fb.unpack_codes(out["codes"], fmt)
        assert np.all(q[2] == 0) and np.all(q[:, 5] == 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_outputs_are_representable(oracle_lib, fmt):
    group = GROUP[fmt]
    W = _rand_w(30, 5 * group, seed=41)
    out = oracle_lib.solve(W, "f32", fmt, group, 6)
    for v in np.concatenate([out["a"], out["b"]]):
        assert fb.representable(fmt, float(v)), (fmt, v)
    s = fb.decode_scales(out["scales"], fmt)
    if fmt == "nvfp4":
        assert np.all(np.isin(s, fb.E4M3_POS_VALS[1:]))
    elif fmt == "int4_bf16":
        assert np.all((fb.bf16_decode(out["scales"]) == s.astype(np.float32)))
    else:
        assert np.all(np.abs(out["scales"].astype(int) - 127) <= 126)


@pytest.mark.parametrize("fmt", ["int4_bf16", "mxint4", "mxfp4", "nvfp4"])
def test_q_is_idempotent(oracle_lib, fmt):
    group = GROUP[fmt]
    W = _rand_w(24, 4 * group, seed=51)
    g = 0.0
    out = oracle_lib.quantize(W, "f32", fmt, group, g=g)
    Qh = _qhat(out, fmt, group).astype(np.float32)
    if fmt != "nvfp4":  # q * d is exact in fp32; NVFP4's d = fl32(s g) has 24 bits
        assert np.array_equal(Qh.astype(np.float64), _qhat(out, fmt, group))
    again = oracle_lib.quantize(Qh, "f32", fmt, group, g=out["g"])
    if fmt == "nvfp4":
        # holds for blocks whose E4M3 scale is normal (>= 2^-6)
        s = fb.decode_scales(out["scales"], fmt)
        keep = np.repeat(s >= 2.0 ** -6, group, axis=1)
        assert keep.mean() > 0.5
        q1 = fb.unpack_codes(out["codes"], fmt)
        q2 = fb.unpack_codes(again["codes"], fmt)
        assert np.array_equal(q1[keep], q2[keep])
    else:
        assert np.array_equal(again["codes"], out["codes"])
        assert np.array_equal(again["scales"], out["scales"])


@pytest.mark.parametrize("fmt", ["int4_bf16", "mxint4", "mxfp4"])
def test_on_grid_weight_is_a_fixed_point(oracle_lib, fmt):
    rng = np.random.default_rng(61)
    group, rows, cols = 32, 10, 128
    if fmt == "mxfp4":
        vals = np.array([v for v in fb.E2M1_TABLE if v != 0])
        q = rng.choice(vals, (rows, cols))
        q[:, ::group] = 6.0  # each group's max sets the shared exponent (m/d = 6)
    else:
        q = rng.integers(-7, 8, (rows, cols)).astype(np.float64)
        q[:, ::group] = 7.0 if fmt == "int4_bf16" else 4.0
    s = 2.0 ** rng.integers(-9, -3, (rows, cols // group))
    if fmt == "int4_bf16":
        s = fb.bf16_decode(np.array(rng.integers(0x3B00, 0x3D00, (rows, cols // group)),
                                    np.uint16)).astype(np.float64)
    W = (q * np.repeat(s, group, axis=1)).astype(np.float32)
    out = oracle_lib.solve(W, "f32", fmt, group, 4)
    assert np.all(out["a"] == 1.0) and np.all(out["b"] == 1.0)
    assert np.all(out["mse"] == 0.0)
    assert np.array_equal(_qhat(out, fmt, group), W.astype(np.float64))


@pytest.mark.parametrize("fmt", FMTS)
def test_mse_trajectory_is_reconstruction_error(oracle_lib, fmt):
    # mse[t] is the error of the synced state after t iterations, recomputed here from
    # the decoded output of an independent quantization at that state
    group = GROUP[fmt]
    W = _rand_w(20, 4 * group, seed=71)
    W64 = W.astype(np.float64)
    T = 5
    full = oracle_lib.solve(W, "f32", fmt, group, T)
    for t in [0, 2, T]:
        st = oracle_lib.solve(W, "f32", fmt, group, t)
        q = oracle_lib.quantize(W, "f32", fmt, group, st["a"], st["b"], st["g"])
        rec = st["a"][:, None].astype(np.float64) * _qhat(q, fmt, group) * \
            st["b"][None, :].astype(np.float64)
        want = np.mean((W64 - rec) ** 2)
        assert abs(full["mse"][t] - want) <= 1e-12 * want
    # mse[0] is plain single-scale RTN (a = b = 1)
    q0 = oracle_lib.quantize(W, "f32", fmt, group)
    assert abs(full["mse"][0] - np.mean((W64 - _qhat(q0, fmt, group)) ** 2)) <= 1e-12 * full["mse"][0]


@pytest.mark.parametrize("fmt", FMTS)
def test_split_objective_never_increases_within_a_step(oracle_lib, fmt):
    group = GROUP[fmt]
    W = _rand_w(32, 6 * group, seed=81)
    W64 = W.astype(np.float64)
    st = oracle_lib.solve(W, "f32", fmt, group, 0)
    a, b, g = st["a"], st["b"], st["g"]

    def obj(av, bv, Qh):
        return np.sum((W64 - av[:, None].astype(np.float64) * Qh * bv[None, :]) ** 2)

    for _ in range(5):
        nxt = oracle_lib.solve(W, "f32", fmt, group, 1, a0=a, b0=b, g0=g)
        Q0 = _qhat(oracle_lib.quantize(W, "f32", fmt, group, a, b, g), fmt, group)
        an = nxt["a"]
        assert obj(an, b, Q0) <= obj(a, b, Q0) * (1 + 1e-12)
        Q1 = _qhat(oracle_lib.quantize(W, "f32", fmt, group, an, b, g), fmt, group)
        assert obj(an, nxt["b"], Q1) <= obj(an, b, Q1) * (1 + 1e-12)
        a, b = an, nxt["b"]


def test_true_mse_descends_once_codes_are_stable(oracle_lib):
    # daiwk notes / trove "Limits": descent is only guaranteed after the grid assignment
    # stops changing; check it on the iterations where no code or scale changed
    qualified = 0
    for fmt in FMTS:
        group = GROUP[fmt]
        W = _rand_w(16, 2 * group, seed=91)
        out = oracle_lib.solve(W, "f32", fmt, group, 25, diag=True)
        for t in range(25):
            if not out["changes"][t].any():
                qualified += 1
                assert out["mse"][t + 1] <= out["mse"][t] * (1 + 1e-12)
    assert qualified > 0


@pytest.mark.parametrize("fmt", ["mxint4", "mxfp4"])
def test_e8m0_gauge_identity(oracle_lib, fmt):
    # with power-of-two scales, a -> 2^k a leaves the codes unchanged and moves each inner
    # scale by 2^-k, so a_i * s_ig is invariant
    W = _rand_w(16, 128, seed=101)
    a = np.array([2.0 ** k for k in np.random.default_rng(3).integers(-3, 4, 16)], np.float32)
    base = oracle_lib.quantize(W, "f32", fmt, 32, a)
    for k in (-1, 1, 5):
        other = oracle_lib.quantize(W, "f32", fmt, 32, (a * 2.0 ** k).astype(np.float32))
        assert np.array_equal(other["codes"], base["codes"])
        assert np.array_equal(other["scales"].astype(int), base["scales"].astype(int) - k)


@pytest.mark.parametrize("fmt", FMTS)
def test_permutation_and_power_of_two_equivariance(oracle_lib, fmt):
    group = GROUP[fmt]
    rows, cols = 20, 4 * group
    W = _rand_w(rows, cols, seed=111)
    T = 4
    base = oracle_lib.solve(W, "f32", fmt, group, T)
    rng = np.random.default_rng(5)
    pr = rng.permutation(rows)
    out = oracle_lib.solve(np.ascontiguousarray(W[pr]), "f32", fmt, group, T)
    assert np.array_equal(out["a"], base["a"][pr])
    assert np.array_equal(out["codes"], base["codes"][pr])
    assert np.array_equal(out["scales"], base["scales"][pr])
    if fmt != "nvfp4":  # NVFP4's g is a whole-tensor max: permutation-invariant as well
        pass
    pg = rng.permutation(cols // group)
    pc = (pg[:, None] * group + np.arange(group)[None, :]).reshape(-1)
    out = oracle_lib.solve(np.ascontiguousarray(W[:, pc]), "f32", fmt, group, T)
    assert np.array_equal(out["b"], base["b"][pc])
    assert np.array_equal(out["scales"], base["scales"][:, pg])
    assert np.allclose(out["mse"], base["mse"], rtol=1e-12, atol=0)
    k = 3
    out = oracle_lib.solve((W * np.float32(2.0 ** k)).astype(np.float32), "f32", fmt, group, T)
    assert np.array_equal(out["codes"], base["codes"])
    assert np.array_equal(out["a"], base["a"]) and np.array_equal(out["b"], base["b"])
    if fmt == "nvfp4":
        assert out["g"] == base["g"] * 2.0 ** k
    else:
        assert np.array_equal(fb.decode_scales(out["scales"], fmt),
                              fb.decode_scales(base["scales"], fmt) * 2.0 ** k)
    assert np.allclose(out["mse"], base["mse"] * 4.0 ** k, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", FMTS)
def test_resume_equals_one_long_run(oracle_lib, fmt):
    group = GROUP[fmt]
    W = _rand_w(16, 4 * group, seed=121)
    full = oracle_lib.solve(W, "f32", fmt, group, 7)
    first = oracle_lib.solve(W, "f32", fmt, group, 3)
    rest = oracle_lib.solve(W, "f32", fmt, group, 4, a0=first["a"], b0=first["b"], g0=first["g"])
    for key in ("a", "b", "codes", "scales"):
        assert np.array_equal(rest[key], full[key])
    assert np.array_equal(np.concatenate([first["mse"][:3], rest["mse"]]), full["mse"])


def test_thread_count_does_not_change_results(oracle_lib):
    W = _rand_w(64, 256, seed=131)
    base = oracle_lib.solve(W, "f32", "mxfp4", 32, 4)
    oracle_lib.set_threads(4)
    try:
        par = oracle_lib.solve(W, "f32", "mxfp4", 32, 4)
    finally:
        oracle_lib.set_threads(1)
    for key in ("a", "b", "codes", "scales", "mse"):
        assert np.array_equal(par[key], base[key])


def test_status_codes(oracle_lib):
    W = _rand_w(4, 64, seed=141)
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.solve(W, "f32", "int4_bf16", 48, 1)  # group not in {16, 32, 64}
    assert e.value.status == 1
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.solve(W[:, :40].copy(), "f32", "int4_bf16", 32, 1)  # cols % group
    assert e.value.status == 1
    bad = W.copy()
    bad[1, 2] = np.nan
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.solve(bad, "f32", "mxfp4", 32, 1)
    assert e.value.status == 3
    with pytest.raises(oracle_lib.OracleError) as e:  # scaled tile overflows
        oracle_lib.solve(W * np.float32(1e30), "f32", "int4_bf16", 32, 1,
                         b0=np.full(64, 1e-30, np.float32))
    assert e.value.status == 4
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.solve(W, "f32", "int4_bf16", 32, 1, a0=-np.ones(4, np.float32))
    assert e.value.status == 1

"""Pins of the oracle's activation quantizer (dq_ref_quantize_act): x = fl32(X * b) per
channel, then the format's group quantizer Q (daiwk notes, "核心公式" eq. 1: the activation
side of the factorized product is X D_b; the flowchart scales the real activations by the
column inverse scales before quantizing them).

Against independent recomputation: the scaled values are formed here with numpy's IEEE
float32 multiply, and every group's scale rule and sampled codes are checked by exact
rational enumeration (qbrute.check_q_output); closed-form bounds on the dequantized error;
special cases (b = None, zero rows, power-of-two b); and every status code."""
import numpy as np
import pytest

import fmt_brute as fb
from cases import adversarial_w
from qbrute import check_q_output

FMTS = ["int4_bf16", "mxint4", "mxfp4", "nvfp4"]
GROUP = {"int4_bf16": 64, "mxint4": 32, "mxfp4": 32, "nvfp4": 16}


def _acts(tokens, cols, seed, outliers=3):
    """Activation-like rows: N(0, 1) with a few channels 20-50x larger."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((tokens, cols)).astype(np.float32)
    ch = rng.choice(cols, size=outliers, replace=False)
    X[:, ch] *= rng.uniform(20, 50, outliers).astype(np.float32)
    return X


def _scaled(X, b):
    return X if b is None else (X * b[None, :].astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("group", [16, 32, 64])
def test_act_quantizer_matches_brute_force_at_ties(oracle_lib, fmt, group):
    # planted rounding ties survive a power-of-two channel scale exactly
    X = adversarial_w(fmt, group, 12, seed=group + 3)
    rng = np.random.default_rng(group)
    b = (2.0 ** rng.integers(-3, 4, X.shape[1])).astype(np.float32)
    out = oracle_lib.quantize_act(X, "f32", fmt, group, b)
    check_q_output(out, _scaled(X, b), fmt, group, 0.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_act_quantizer_with_format_scales_matches_brute_force(oracle_lib, fmt):
    group = GROUP[fmt]
    rng = np.random.default_rng(31)
    X = _acts(10, 4 * group, seed=32)
    b = np.array([fb.project(fmt, v) for v in rng.uniform(0.05, 4, 4 * group)], np.float32)
    out = oracle_lib.quantize_act(X, "f32", fmt, group, b)
    check_q_output(out, _scaled(X, b), fmt, group, 0.0)
    if fmt == "nvfp4":  # a given tensor scale is used as is
        out = oracle_lib.quantize_act(X, "f32", fmt, group, b, g=0.0123)
        assert out["g"] == np.float32(0.0123)
        check_q_output(out, _scaled(X, b), fmt, group, 0.0123)


@pytest.mark.parametrize("fmt", FMTS)
def test_act_quantizer_bf16_input(oracle_lib, fmt):
    group = GROUP[fmt]
    X32 = _acts(8, 2 * group, seed=41)
    Xb = fb.torch_bf16(X32).astype(np.float32)  # the values the bf16 bits hold
    bits = (Xb.view(np.uint32) >> 16).astype(np.uint16)
    b = np.linspace(0.5, 2.0, 2 * group).astype(np.float32)
    b = np.array([fb.project(fmt, float(v)) for v in b], np.float32)
    got = oracle_lib.quantize_act(bits, "bf16", fmt, group, b)
    want = oracle_lib.quantize_act(Xb, "f32", fmt, group, b)
    for k in ("codes", "scales"):
        assert np.array_equal(got[k], want[k]), k
    check_q_output(got, _scaled(Xb, b), fmt, group, 0.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantized_error_bound(oracle_lib, fmt):
    # |x - q d| <= half the local grid step times d wherever the code is not saturated
    # (INT4/BF16 never saturates: its scale keeps |x / d| <= 7.03; MXINT4 saturates at 7,
    # since its shared exponent puts the group max at 4..8 d; E2M1 at 6)
    group = GROUP[fmt]
    X = _acts(16, 4 * group, seed=51)
    b = np.array([fb.project(fmt, float(v)) for v in np.linspace(0.3, 3, 4 * group)], np.float32)
    out = oracle_lib.quantize_act(X, "f32", fmt, group, b)
    x = _scaled(X, b).astype(np.float64)
    deq = fb.dequant(out["codes"], out["scales"], fmt, group, out["g"])
    d = np.repeat(fb.divisors(out["scales"], fmt, out["g"]), group, axis=1)
    q = fb.unpack_codes(out["codes"], fmt)
    err = np.abs(x - deq)
    if fmt == "int4_bf16":
        assert np.all(err <= 0.5 * d * (1 + 1e-12))
    elif fmt == "mxint4":
        assert np.all((err <= 0.5 * d * (1 + 1e-12)) | (np.abs(q) == 7))
        assert np.all(err <= d)  # |x| < 8 d
    else:
        step = np.where(np.abs(q) < 2, 0.5, np.where(np.abs(q) < 4, 1.0, 2.0))
        assert np.all(err <= 0.5 * step * d * (1 + 1e-12) + np.where(np.abs(q) == 6, np.inf, 0))


def test_special_cases(oracle_lib):
    X = _acts(6, 128, seed=61)
    X[2] = 0.0
    for fmt in FMTS:
        group = GROUP[fmt]
        one = oracle_lib.quantize_act(X, "f32", fmt, group, None)
        ones = oracle_lib.quantize_act(X, "f32", fmt, group, np.ones(128, np.float32))
        for k in ("codes", "scales"):
            assert np.array_equal(one[k], ones[k]), (fmt, k)
        assert np.all(one["codes"][2] == 0)
        assert np.all(fb.decode_scales(one["scales"], fmt)[2] == 1.0)
    # E8M0 formats: scaling every channel by 2^k shifts every shared exponent by k (away from
    # the clamp) and keeps every code
    for fmt in ("mxint4", "mxfp4"):
        base = oracle_lib.quantize_act(X, "f32", fmt, 32, None)
        sh = oracle_lib.quantize_act(X, "f32", fmt, 32, np.full(128, 8.0, np.float32))
        assert np.array_equal(base["codes"], sh["codes"])
        nz = np.abs(X).reshape(6, 4, 32).max(-1) > 0
        assert np.all((sh["scales"].astype(int) - base["scales"].astype(int))[nz] == 3)


def test_act_status_codes(oracle_lib):
    X = _acts(4, 64, seed=71)
    with pytest.raises(oracle_lib.OracleError) as e:
        bad = X.copy()
        bad[1, 5] = np.nan
        oracle_lib.quantize_act(bad, "f32", "mxfp4", 32)
    assert e.value.status == 3
    with pytest.raises(oracle_lib.OracleError) as e:  # X * b overflows fp32
        oracle_lib.quantize_act(X * np.float32(1e30), "f32", "mxfp4", 32,
                                np.full(64, 1e20, np.float32))
    assert e.value.status == 4
    with pytest.raises(oracle_lib.OracleError) as e:
        b = np.ones(64, np.float32)
        b[3] = 0.0
        oracle_lib.quantize_act(X, "f32", "mxfp4", 32, b)
    assert e.value.status == 1
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.quantize_act(X, "f32", "mxfp4", 48)
    assert e.value.status == 1

"""CPU checks of the HIP library's codec header (dual_scale_w4a4_amd/csrc/dq_device.h),
built for the host: rounding to bf16 / E4M3 / E2M1, the projections of the outer scales and
the per-group quantizer, against brute-force enumeration, torch's conversions and the oracle.
These run without a GPU, so a codec bug shows up before any kernel launch."""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

import fmt_brute as fb
from cases import adversarial_w, rand_w

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libdq_codec_host.so")
SRC = [os.path.join(HERE, "codec_host.hip"),
       os.path.join(os.path.dirname(HERE), "dual_scale_w4a4_amd", "csrc", "dq_device.h"),
       os.path.join(os.path.dirname(HERE), "dual_scale_w4a4_amd", "csrc", "dq_internal.h")]


@pytest.fixture(scope="module")
def H():
    # DQ_CODEC_HOST_LIB: load another build of codec_host.hip instead (for example one built
    # with the host sanitizers)
    if os.environ.get("DQ_CODEC_HOST_LIB"):
        return ctypes.CDLL(os.environ["DQ_CODEC_HOST_LIB"])
    os.makedirs(BUILD, exist_ok=True)
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(s) for s in SRC):
        tmp = f"{LIB}.tmp{os.getpid()}"  # parallel test workers may build at once
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-fPIC", "-shared", "-ffp-contract=off", SRC[0], "-o", tmp],
                       check=True, capture_output=True)
        os.replace(tmp, LIB)
    return ctypes.CDLL(LIB)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _map(H, name, x, out_dtype=np.float32):
    x = np.ascontiguousarray(x)
    y = np.zeros(x.shape, out_dtype)
    getattr(H, name)(_p(x), _p(y), ctypes.c_int64(x.size))
    return y


def test_bf16_rne_all_upper_halves(H):
    hi = np.arange(0, 0x7F7F, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234], np.uint32)
    x = (hi[:, None] << 16 | lows[None, :]).reshape(-1).view(np.float32)
    assert np.array_equal(_map(H, "h_bf16_rne", x).astype(np.float64), fb.torch_bf16(x))


def test_e4m3_rne_sat_against_enumeration(H):
    pos = fb.E4M3_POS_VALS
    vals = set(pos.tolist()) | set(((pos[1:] + pos[:-1]) / 2).tolist()) | {456.0, 464.0, 1e6, 1e-30}
    x = np.array(sorted(vals), np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))])
    rng = np.random.default_rng(0)
    x = np.concatenate([x, np.exp(rng.uniform(-12, 7, 4000)).astype(np.float32)])
    got = _map(H, "h_e4m3_rne_sat", x)
    want = np.array([fb.e4m3_nearest_sat(float(v)) for v in x])
    assert np.array_equal(got.astype(np.float64), want)
    codes = _map(H, "h_e4m3_bits", pos[1:].astype(np.float32), np.uint32)
    assert np.array_equal(codes, np.arange(1, 0x7F))


def test_e2m1_mag_against_enumeration(H):
    rng = np.random.default_rng(1)
    grid = np.array(sorted(set(abs(v) for v in fb.E2M1_TABLE)))
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([grid, mids, rng.uniform(0, 8, 20000), [7.0, 7.99, 1e-40, 0.0]]).astype(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(8)), np.nextafter(x, np.float32(0))])
    x = x[x < 8]
    assert np.array_equal(_map(H, "h_e2m1_mag", x).astype(np.float64), fb.e2m1_nearest(x.astype(np.float64)))


@pytest.mark.parametrize("fmt,fid", [("int4_bf16", 0), ("mxfp4", 2), ("nvfp4", 3)])
def test_projections_against_enumeration(H, fmt, fid):
    rng = np.random.default_rng(2)
    v = list(np.exp(rng.uniform(math.log(1e-4), math.log(1e4), 400)))
    if fmt == "int4_bf16":
        base = fb.bf16_decode(rng.integers(0x3000, 0x5000, 200).astype(np.uint16)).astype(np.float64)
        step = np.ldexp(1.0, np.frexp(base)[1] - 8)
        m = base + step / 2  # exact midpoints
        v += list(m) + [math.nextafter(t, 0) for t in m] + [math.nextafter(t, 9) for t in m]
        v += [1e-300, 1e-39, 3.5e38, 1e300]
    elif fmt == "mxfp4":
        m = 1.5 * np.ldexp(1.0, np.arange(-128, 129))
        v += list(m) + [math.nextafter(t, 0) for t in m] + [1e-300, 1e300]
    else:
        pos = fb.E4M3_POS_VALS[1:]
        m = (pos[1:] + pos[:-1]) / 2
        v += list(m) + [math.nextafter(t, 0) for t in m] + [math.nextafter(t, 999) for t in m]
        v += [1e-7, 1000.0]
    x = np.array(v, np.float64)
    y = np.zeros(len(x), np.float32)
    H.h_project(ctypes.c_int(fid), _p(x), _p(y), ctypes.c_int64(len(x)))
    want = np.array([fb.project(fmt, float(t)) for t in x])
    assert np.array_equal(y.astype(np.float64), want)


def test_recip32_is_correctly_rounded(H):
    rng = np.random.default_rng(3)
    x = np.exp(rng.uniform(-80, 80, 20000)).astype(np.float32)
    want = (np.float32(1.0) / x).astype(np.float32)  # numpy: IEEE division
    assert np.array_equal(_map(H, "h_recip32", x), want)


@pytest.mark.parametrize("fmt,fid,group", [("int4_bf16", 0, 32), ("mxint4", 1, 32), ("mxfp4", 2, 32),
                                            ("nvfp4", 3, 16), ("int4_bf16", 0, 64), ("nvfp4", 3, 64)])
def test_group_quantizer_matches_oracle(H, oracle_lib, fmt, fid, group):
    rng = np.random.default_rng(4)
    for W, a, b in [
        (adversarial_w(fmt, group, 60, seed=5), None, None),
        (rand_w(50, 8 * group, seed=6, outliers=9),
         rng.uniform(0.1, 5, 50).astype(np.float32), rng.uniform(0.1, 5, 8 * group).astype(np.float32)),
    ]:
        rows, cols = W.shape
        A = np.ones(rows, np.float32) if a is None else a
        B = np.ones(cols, np.float32) if b is None else b
        X = fb.scaled_tile(W, A, B)
        ref = oracle_lib.quantize(W, "f32", fmt, group, a, b)
        q = np.zeros((rows, cols), np.float32)
        sc = np.zeros((rows, cols // group), np.uint32)
        H.h_quantize(ctypes.c_int(fid), _p(X), ctypes.c_int64(rows), ctypes.c_int64(cols),
                     ctypes.c_int(group), ctypes.c_float(ref["g"] if fmt == "nvfp4" else 1.0),
                     _p(q), _p(sc))
        assert np.array_equal(q.astype(np.float64), fb.unpack_codes(ref["codes"], fmt))
        assert np.array_equal(sc, ref["scales"].astype(np.uint32))


def test_div7_is_the_correctly_rounded_quotient(H):
    # the argument (a fractional part k/7 never near a rounding midpoint) does not depend on
    # the exponent except where m / 7 is subnormal: every subnormal m, every m whose quotient
    # is subnormal or at the boundary, and a few normal binades including the largest
    H.h_div7_mismatches.restype = ctypes.c_int64
    for e0, e1 in [(0, 3), (126, 128), (200, 200), (254, 254)]:
        assert H.h_div7_mismatches(e0, e1) == 0, (e0, e1)


def test_int4_quotient_rounding_at_ties_with_inexact_reciprocal(H):
    # every bf16 significand at several exponents, plus subnormal bf16 divisors
    sig = np.arange(128, 256, dtype=np.float64)
    d = np.concatenate([sig * 2.0 ** e for e in (-140, -133, -127, -107, -20, -7, 0, 9, 60, 110)])
    d = d[(d >= 2.0 ** -133) & (d < 2.0 ** 120)].astype(np.float32)
    H.h_rne_quotient_mismatches.restype = ctypes.c_int64
    assert H.h_rne_quotient_mismatches(_p(d), ctypes.c_int64(d.size)) == 0


def test_double_quotient_codes_at_boundaries(H):
    H.h_code64_mismatches.restype = ctypes.c_int64
    sig = np.arange(128, 256, dtype=np.float64)
    # INT4 divisors: bf16 values, normal and subnormal (down to the 2^-133 floor)
    d = np.concatenate([sig * 2.0 ** e for e in (-140, -133, -127, -107, -20, -7, 0, 9, 60, 110)])
    d = d[(d >= 2.0 ** -133) & (d < 2.0 ** 120)].astype(np.float32)
    assert H.h_code64_mismatches(0, _p(d), ctypes.c_int64(d.size)) == 0
    # NVFP4 divisors: fl32(s * g), s an E4M3 value, g an arbitrary fp32 tensor scale
    rng = np.random.default_rng(5)
    s = fb.E4M3_POS_VALS[fb.E4M3_POS_VALS > 0]
    g = np.concatenate([np.exp(rng.uniform(-30, 30, 40)), [2.0 ** -126, 1.0, 1.0 / 3.0]])
    d = (s[None, :].astype(np.float32) * g[:, None].astype(np.float32)).reshape(-1)
    d = d[(d > 0) & np.isfinite(d)].astype(np.float32)
    assert H.h_code64_mismatches(3, _p(d), ctypes.c_int64(d.size)) == 0


def test_nvfp4_scale_quotient_by_fp64_reciprocal():
    # NVFP4's u = fl32(mx / fl32(6 g)) is taken on the GPU as fl32(mx * r6) with
    # r6 = 1 / fl32(6 g) correctly rounded in fp64 (both fp64 operations are IEEE there, as
    # here): equal for random values over the whole range, for mx next to multiples of
    # fl32(6 g) by an E4M3 value (the quotients that matter most) and for subnormal mx
    rng = np.random.default_rng(13)
    six = np.float32(6.0)
    g = np.concatenate([np.exp(rng.uniform(-80, 80, 300)), [1.0, 1.0 / 3.0, 0.0071, 2.0 ** -126]])
    sixg = (six * g.astype(np.float32)).astype(np.float32)
    sixg = sixg[np.isfinite(sixg) & (sixg > 0)]
    s = fb.E4M3_POS_VALS[fb.E4M3_POS_VALS > 0]
    for sg in sixg:
        r6 = 1.0 / np.float64(sg)
        mx = np.concatenate([
            (s * np.float64(sg)).astype(np.float32),
            (rng.uniform(0, 1, 400) * 2.0 ** rng.integers(-149, 128, 400)).astype(np.float32)])
        mx = np.concatenate([mx, np.nextafter(mx, np.float32(np.inf)), np.nextafter(mx, np.float32(0))])
        mx = mx[np.isfinite(mx) & (mx > 0)]
        with np.errstate(over="ignore", under="ignore"):
            want = (mx.astype(np.float64) / np.float64(sg)).astype(np.float32)
            got = (mx.astype(np.float64) * r6).astype(np.float32)
        assert np.array_equal(want, got), (sg, mx[want != got][:4])


def test_nvfp4_odd_quotient_codes_at_boundaries(H):
    # the fp32 NVFP4 codes of the activation quantizer and the two-sweep pass: divisors
    # fl32(s g) for every positive E4M3 value s and tensor scales g across the range, plus
    # random fp32 divisors, all within [2^-100, 2^100] where that path is taken
    H.h_nv_odd_mismatches.restype = ctypes.c_int64
    rng = np.random.default_rng(11)
    s = fb.E4M3_POS_VALS[fb.E4M3_POS_VALS > 0]
    g = np.concatenate([np.exp(rng.uniform(-60, 60, 40)), [2.0 ** -90, 1.0, 1.0 / 3.0, 0.0071]])
    d = (s[None, :].astype(np.float32) * g[:, None].astype(np.float32)).reshape(-1)
    r = (rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-100, 100, 3000)).astype(np.float32)
    d = np.concatenate([d, r])
    d = d[(d >= 2.0 ** -100) & (d <= 2.0 ** 100)].astype(np.float32)
    assert d.size > 8000
    assert H.h_nv_odd_mismatches(_p(d), ctypes.c_int64(d.size)) == 0


@pytest.mark.parametrize("fmt,fid", [("int4_bf16", 0), ("nvfp4", 3)])
@pytest.mark.parametrize("group", [16, 32, 64])
def test_double_quotient_group_quantizer_matches_oracle(H, oracle_lib, fmt, fid, group):
    # the codes as the two-sweep pass and the activation quantizer form them (code64, with
    # INT4's clamp where the scale is a subnormal bf16 value), on rows with planted ties,
    # zero groups, subnormal groups (subnormal INT4 scales) and outliers
    W = adversarial_w(fmt, group, 60, seed=group + 7)
    W[7, :group] = (np.linspace(-1, 1, group) * 2.2e-39).astype(np.float32)  # subnormal scale
    ref = oracle_lib.quantize(W, "f32", fmt, group, None, None)
    qr = fb.unpack_codes(ref["codes"], fmt)
    H.h_group_code64.restype = None
    rows, cols = W.shape
    for i in range(rows):
        for k in range(cols // group):
            x = np.ascontiguousarray(W[i, k * group:(k + 1) * group])
            q = np.zeros(group)
            sc = np.zeros(1, np.uint32)
            H.h_group_code64(ctypes.c_int(fid), _p(x), ctypes.c_int(group),
                             ctypes.c_float(ref["g"] if fmt == "nvfp4" else 1.0), _p(q), _p(sc))
            assert sc[0] == int(ref["scales"][i, k]), (i, k)
            assert np.array_equal(q, qr[i, k * group:(k + 1) * group]), (i, k, q, qr[i, k * group:(k + 1) * group])

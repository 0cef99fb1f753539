"""GPU parity of the activation quantizer (dq_quantize_act) against the oracle: a single Q
pass on x = fl32(X * b), so codes, inner scales and the NVFP4 tensor scale must be
bit-identical. Covers every format and group size, bf16 and fp32 inputs, ragged channel and
token counts, planted rounding ties, zero rows, group scales outside the range where the
hardware FP4 conversion is used, the full-size Llama-3.1-8B MLP inputs, and the error
statuses."""
import numpy as np
import pytest

import workloads
import fmt_brute as fb
from cases import adversarial_w
from parity import host, to_device

pytestmark = pytest.mark.gpu

FMTS = ["int4_bf16", "mxint4", "mxfp4", "nvfp4"]


@pytest.fixture(scope="module")
def dq():
    import torch

    assert torch.cuda.is_available()
    import dual_scale_w4a4_amd

    dual_scale_w4a4_amd.lib()
    return dual_scale_w4a4_amd


def _bvec(b):
    return None if b is None else to_device(np.ascontiguousarray(b, np.float32), "f32")


def _check(dq, oracle, X, dtype, fmt, group, b, g=0.0, name=""):
    print(f"[act] {name} {fmt} G={group} {dtype} {X.shape} g={g}", flush=True)
    ref = oracle.quantize_act(X, dtype, fmt, group, b, g)
    got = dq.quantize_act(to_device(X, dtype), fmt, group, _bvec(b), g)
    codes, scales = host(got["codes"]), host(got["scales"])
    if fmt == "int4_bf16":
        scales = scales.view(np.uint16)
    bad = np.argwhere(codes != ref["codes"])
    assert bad.size == 0, (name, fmt, group, bad[:5])
    assert np.array_equal(scales, ref["scales"]), (name, fmt, group)
    if fmt == "nvfp4":
        assert np.float32(host(got["g"])[0]) == np.float32(ref["g"]), (host(got["g"]), ref["g"])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("group", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_act_matches_oracle_ragged(dq, oracle_lib, fmt, group, dtype):
    # 1088 channels: one full 1024-channel tile and a partial one; 67 tokens: a ragged chunk
    X = workloads.activations(67, 1088, seed=group, dtype=dtype)
    b = workloads.act_column_scales(1088, seed=group)
    _check(dq, oracle_lib, X, dtype, fmt, group, b, name="ragged")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("group", [16, 32, 64])
def test_act_ties_and_special_rows(dq, oracle_lib, fmt, group):
    X = adversarial_w(fmt, group, 40, seed=group + 7)  # ties, zero groups, subnormals
    X[3] = 0.0
    rng = np.random.default_rng(group)
    b = (2.0 ** rng.integers(-3, 4, X.shape[1])).astype(np.float32)
    _check(dq, oracle_lib, X, "f32", fmt, group, b, name="ties")
    _check(dq, oracle_lib, X, "f32", fmt, group, None, name="ties-b=1")


def test_act_nvfp4_given_tensor_scale(dq, oracle_lib):
    X = workloads.activations(50, 2048, seed=5)
    b = workloads.act_column_scales(2048, seed=5)
    _check(dq, oracle_lib, X, "bf16", "nvfp4", 16, b, g=0.0071, name="given-g")


def _nvfp4_tie_rows(g, rows, cols, seed):
    """Rows whose 16-element groups each fix an E4M3 scale s (their first element is the one
    of fl32(s * fl32(6 g)) and its neighbours with u = s exactly) and put the other elements
    on E2M1 decision points times d = fl32(s g), or one fp32 step either side, with random
    signs."""
    rng = np.random.default_rng(seed)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    svals = fb.E4M3_POS_VALS[(fb.E4M3_POS_VALS >= 2.0 ** -6) & (fb.E4M3_POS_VALS <= 448.0)]
    g = np.float32(g)
    sixg = np.float32(6.0 * np.float64(g))
    X = np.zeros((rows, cols), np.float32)
    for i in range(rows):
        for k in range(cols // 16):
            mx = None
            while mx is None:  # some s are no fl32(mx / fl32(6 g)): draw another
                s = np.float32(rng.choice(svals))
                mx0 = np.float32(np.float64(s) * np.float64(sixg))
                cands = [mx0, np.nextafter(mx0, np.float32(np.inf)), np.nextafter(mx0, np.float32(0))]
                ok = [c for c in cands if np.float32(np.float64(c) / np.float64(sixg)) == s]
                mx = ok[0] if ok else None
            d = np.float32(np.float64(s) * np.float64(g))
            base = (mids[rng.integers(0, 7, 15)] * np.float64(d)).astype(np.float32)
            step = rng.integers(-1, 2, 15)
            near = np.where(step > 0, np.nextafter(base, np.float32(np.inf)),
                            np.where(step < 0, np.nextafter(base, np.float32(0)), base))
            sign = np.where(rng.integers(0, 2, 15) == 1, -1, 1).astype(np.float32)
            X[i, 16 * k] = mx
            X[i, 16 * k + 1:16 * k + 16] = sign * near
    return X


def test_act_nvfp4_ties_at_non_power_of_two_scales(dq, oracle_lib):
    # With g = 3/256 the decision points times d are fp32 values (exact ties); with g =
    # 0.0071 they are not, and the elements lie within an ulp of a tie on either side. Row 5
    # is scaled up so that its scale saturates at 448 (quotients beyond 8, clamped before
    # the fp32 quotient), and the last call has d below 2^-100, which takes the double
    # quotient.
    for g in (3.0 / 256.0, 0.0071):
        X = _nvfp4_tie_rows(g, 24, 512, seed=int(g * 1e4))
        X[5] *= np.float32(64.0)
        _check(dq, oracle_lib, X, "f32", "nvfp4", 16, None, g=g, name=f"nv-ties g={g}")
    g = float(np.float32(1.3 * 2.0 ** -110))
    X = _nvfp4_tie_rows(g, 8, 256, seed=3)
    _check(dq, oracle_lib, X, "f32", "nvfp4", 16, None, g=g, name="nv-ties tiny g")


def test_act_group_scales_outside_the_conversion_range(dq, oracle_lib):
    # MXFP4 group scales below 2^-100 and above 2^20 take the exact fp32 path, in the same
    # waves as ordinary groups
    rng = np.random.default_rng(9)
    X = rng.standard_normal((32, 2048)).astype(np.float32)
    X[::3, 64:96] *= np.float32(2.0 ** -110)
    X[1::3, 128:160] *= np.float32(2.0 ** 30)
    X[2, :32] = np.float32(2.0 ** -140)  # subnormal
    for fmt in FMTS:
        _check(dq, oracle_lib, X, "f32", fmt, 32, None, name="extreme")


@pytest.mark.parametrize("which", ["up", "down"])
def test_act_full_size_llama8b_mlp_inputs(dq, oracle_lib, which):
    X, b = workloads.act_inputs(which)
    _check(dq, oracle_lib, X, "bf16", "mxfp4", 32, b, name=f"8192 tokens {which}")
    if which == "up":
        _check(dq, oracle_lib, X, "bf16", "nvfp4", 16, b, name=f"8192 tokens {which}")


def test_act_error_statuses(dq):
    import torch

    X = workloads.activations(16, 256, seed=3, dtype="f32")
    bad = X.copy()
    bad[4, 17] = np.nan
    with pytest.raises(dq.DQError) as e:
        dq.quantize_act(to_device(bad, "f32"), "mxfp4", 32)
    assert e.value.status == 3
    bad[4, 17] = np.inf
    with pytest.raises(dq.DQError) as e:
        dq.quantize_act(to_device(bad, "f32"), "nvfp4", 16)  # through the amax pass
    assert e.value.status == 3
    with pytest.raises(dq.DQError) as e:  # X * b overflows
        dq.quantize_act(to_device(X * np.float32(1e30), "f32"), "int4_bf16", 32,
                        _bvec(np.full(256, 1e20, np.float32)))
    assert e.value.status == 4
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dq.DQError) as e:
        dq.quantize_act(to_device(X, "f32"), "mxfp4", 32, workspace=ws)
    assert e.value.status == 5
    ws = torch.empty(dq.act_workspace_bytes(16, 256, "mxfp4", 32), dtype=torch.uint8, device="cuda")
    x = dq.quantize_act(to_device(X, "f32"), "mxfp4", 32, workspace=ws)
    y = dq.quantize_act(to_device(X, "f32"), "mxfp4", 32)
    assert np.array_equal(host(x["codes"]), host(y["codes"]))


def test_act_async_matches_blocking_and_collects_status(dq):
    import torch

    X, b = workloads.act_inputs("up")
    X = X[:300]
    Xd = to_device(X, "bf16")
    bd = _bvec(b)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for fmt, group in (("mxfp4", 32), ("nvfp4", 16), ("int4_bf16", 64)):
        want = dq.quantize_act(Xd, fmt, group, bd)
        codes = torch.empty_like(want["codes"])
        scales = torch.empty_like(want["scales"])
        gout = torch.zeros(1, dtype=torch.float32, device="cuda")
        dq.quantize_act_async(Xd, fmt, group, codes, scales, status, b=bd, gout=gout)
        torch.cuda.synchronize()
        assert np.array_equal(host(codes), host(want["codes"])), fmt
        assert np.array_equal(host(scales), host(want["scales"])), fmt
        if fmt == "nvfp4":
            assert host(gout)[0] == host(want["g"])[0]
    assert int(host(status)[0]) == 0
    bad = X[:32].copy()
    bad[3, 5] = 0x7FC0  # a bf16 NaN
    Bd = to_device(bad, "bf16")
    out = dq.quantize_act(to_device(X[:32], "bf16"), "mxfp4", 32, bd)
    dq.quantize_act_async(Bd, "mxfp4", 32, out["codes"], out["scales"], status, b=bd)
    torch.cuda.synchronize()
    assert int(host(status)[0]) & 1


def _projected_b(fmt, cols, seed):
    """Column inverse scales drawn as the solver returns them: uniform(0.05, 4) values
    projected onto the format's outer scale set (bf16 values for INT4_BF16, E4M3 values for
    NVFP4), so that most products X * b are inexact in fp32."""
    rng = np.random.default_rng(seed)
    return np.array([fb.project(fmt, float(v)) for v in rng.uniform(0.05, 4.0, cols)],
                    np.float32)


def _inexact_products(X, b):
    exact = X.astype(np.float64) * b[None, :].astype(np.float64)
    return int(np.count_nonzero(exact != (X * b[None, :]).astype(np.float64)))


@pytest.mark.parametrize("fmt,group", [("int4_bf16", 32), ("int4_bf16", 64), ("nvfp4", 16)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_act_with_the_solvers_scale_sets(dq, oracle_lib, fmt, group, dtype):
    X = workloads.activations(67, 1088, seed=group + 3, dtype=dtype)
    b = _projected_b(fmt, 1088, seed=group)
    assert np.mean(np.log2(b) != np.round(np.log2(b))) > 0.5  # mostly not powers of two
    if dtype == "f32":  # bf16 X times a bf16 or E4M3 b is exact in fp32 (<= 16 bits)
        assert _inexact_products(X, b) > X.size // 4
    _check(dq, oracle_lib, X, dtype, fmt, group, b, name="projected b")
    if fmt == "nvfp4":
        _check(dq, oracle_lib, X, dtype, fmt, group, b, g=0.0071, name="projected b, given g")


@pytest.mark.parametrize("fmt,group", [("int4_bf16", 64), ("nvfp4", 16), ("mxfp4", 32)])
def test_act_with_b_from_a_gpu_solve(dq, oracle_lib, fmt, group):
    # the consumer chain: the solver's column scales of a weight with these input channels
    W = workloads.config5_layer(2, scale_down=4, only=("up",))[0].W[:, :1024]
    sol = dq.solve(to_device(np.ascontiguousarray(W), "bf16"), fmt, group, 6)
    b = host(sol["b"])
    X = workloads.activations(40, 1024, seed=11)
    _check(dq, oracle_lib, X, "bf16", fmt, group, b, name=f"b of a {fmt} solve")


def _tie_targets(fmt, group, rows, cols, rng, g=1.0):
    """Scaled activations x with every group's scale fixed by its first element and the
    other elements on the code grid's decision points times the divisor d, or one fp32 step
    either side (INT4_BF16: d a bf16 value, x_max = 7 d, ties at (k + 1/2) d)."""
    if fmt == "nvfp4":
        return _nvfp4_tie_rows(g, rows, cols, seed=int(rng.integers(1 << 30)))
    x = np.zeros((rows, cols), np.float32)
    for i in range(rows):
        for k in range(cols // group):
            d = fb.bf16_decode(np.array([rng.integers(0x3A00, 0x3F00)], np.uint16))[0]
            ks = rng.integers(-7, 7, group - 1) + 0.5
            base = (ks * np.float64(d)).astype(np.float32)
            step = rng.integers(-1, 2, group - 1)
            near = np.where(step > 0, np.nextafter(base, np.float32(np.inf)),
                            np.where(step < 0, np.nextafter(base, np.float32(-np.inf)), base))
            x[i, k * group] = np.float32(7.0 * np.float64(d)) * np.float32(rng.choice([-1, 1]))
            x[i, k * group + 1:(k + 1) * group] = near
    return x


def _unscale(x, b):
    """fp32 X with fl32(X * b) == x where one exists, preferring an X whose exact product
    is not x (so the tie comes out of a rounded product); else the nearest one."""
    X0 = (x.astype(np.float64) / b[None, :].astype(np.float64)).astype(np.float32)
    cands = [X0]
    lo = hi = X0
    for _ in range(3):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        cands += [lo, hi]
    best = X0.copy()
    score = np.full(x.shape, 3, np.int8)  # 0: tie from an inexact product, 1: exact one
    bb = b[None, :].astype(np.float64)
    for c in cands:
        prod = c.astype(np.float64) * bb
        hit = (prod.astype(np.float32) == x)
        s = np.where(hit & (prod != x.astype(np.float64)), 0, np.where(hit, 1, 3)).astype(np.int8)
        take = s < score
        best = np.where(take, c, best)
        score = np.minimum(score, s)
    return best, score


@pytest.mark.parametrize("fmt,group", [("int4_bf16", 32), ("int4_bf16", 64), ("nvfp4", 16)])
def test_act_ties_after_an_inexact_product(dq, oracle_lib, fmt, group):
    # x = fl32(X * b) lands on a code decision point (or one step beside it) although the
    # exact product X * b does not: the quantizer must take the tie from the rounded product
    rng = np.random.default_rng(group + 100)
    cols = 512
    b = _projected_b(fmt, cols, seed=group + 1)
    for g in ((3.0 / 256.0, 0.0071) if fmt == "nvfp4" else (0.0,)):
        x = _tie_targets(fmt, group, 24, cols, rng, g=g)
        X, score = _unscale(x, b)
        assert np.mean(score == 0) > 0.5, np.mean(score == 0)
        got_x = (X * b[None, :]).astype(np.float32)
        assert np.mean(got_x == x) > 0.8
        _check(dq, oracle_lib, X, "f32", fmt, group, b, g=g, name=f"inexact ties g={g}")

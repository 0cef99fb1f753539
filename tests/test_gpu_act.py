"""GPU parity of the activation quantizer (dq_quantize_act) against the oracle: a single Q
pass on x = fl32(X * b), so codes, inner scales and the NVFP4 tensor scale must be
bit-identical. Covers every format and group size, bf16 and fp32 inputs, ragged channel and
token counts, planted rounding ties, zero rows, group scales outside the range where the
hardware FP4 conversion is used, the full-size Llama-3.1-8B MLP inputs, and the error
statuses."""
import numpy as np
import pytest

import workloads
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

"""GPU parity of one Q pass (dq_quantize) against the oracle: codes, inner scales and the
NVFP4 tensor scale must be bit-identical for every format, group size and weight dtype, on
random and adversarial inputs (exact rounding ties, zero groups, subnormals, outliers,
ragged column tiles)."""
import numpy as np
import pytest

from cases import adversarial_w, rand_w
from parity import host, scales_np, to_device

pytestmark = pytest.mark.gpu

FMTS = ["int4_bf16", "mxint4", "mxfp4", "nvfp4"]


@pytest.fixture(scope="module")
def dq():
    import torch

    assert torch.cuda.is_available()
    import dual_scale_w4a4_amd

    dual_scale_w4a4_amd.lib()
    return dual_scale_w4a4_amd


def _to_bf16_bits(W32):
    u = W32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _check(dq, oracle_lib, W, dtype, fmt, group, a=None, b=None, g=0.0, name=""):
    print(f"[quantize] {name} {fmt} G={group} {dtype} {W.shape}", flush=True)
    gpu = dq.quantize(to_device(W, dtype), fmt, group, a, b, g)
    ref = oracle_lib.quantize(W, dtype, fmt, group, a, b, g)
    assert np.array_equal(host(gpu["codes"]), ref["codes"]), name
    assert np.array_equal(scales_np(gpu["scales"], fmt), ref["scales"]), name
    if fmt == "nvfp4":
        assert host(gpu["g"])[0] == np.float32(ref["g"]), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("group", [16, 32, 64])
@pytest.mark.parametrize("fmt", FMTS)
def test_adversarial_bit_exact(dq, oracle_lib, fmt, group, dtype):
    W = adversarial_w(fmt, group, 45, seed=group + 7)
    if dtype == "bf16":
        W = _to_bf16_bits(W)
    _check(dq, oracle_lib, W, dtype, fmt, group, name="adversarial")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_tiles_with_scales_bit_exact(dq, oracle_lib, fmt, dtype):
    rng = np.random.default_rng(3)
    rows, cols = 37, 1056  # two full 512-column tiles and a 32-column tail
    W = rand_w(rows, cols, seed=5, dtype=dtype, outliers=11)
    a = rng.uniform(0.2, 4.0, rows).astype(np.float32)  # arbitrary positive scales
    b = rng.uniform(0.2, 4.0, cols).astype(np.float32)
    _check(dq, oracle_lib, W, dtype, fmt, 16, a, b, name="ragged")
    if fmt == "nvfp4":
        _check(dq, oracle_lib, W, dtype, fmt, 16, a, b, g=3.1e-5, name="given g")


def test_workload_shapes_bit_exact(dq, oracle_lib):
    import workloads

    for w in workloads.reduced(3) + workloads.reduced(4) + workloads.reduced(2):
        _check(dq, oracle_lib, w.W, w.dtype, w.fmt, w.group, name=w.name)

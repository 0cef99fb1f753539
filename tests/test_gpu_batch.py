"""GPU tests of the batch solve (dq_solve_batch): every matrix of a batch must come out
exactly as an individual dq_solve of it (same kernels, same order of operations, only the
launches shared), for a decoder layer's seven matrices, NVFP4 with fixed and per-pass tensor
scales, more matrices than one launch takes, and (MX formats, where the individual solve takes
the single-sweep path) against the single-sweep results."""
import numpy as np
import pytest

import workloads
from cases import rand_w
from parity import host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dq():
    import torch

    assert torch.cuda.is_available()
    import dual_scale_w4a4_amd

    dual_scale_w4a4_amd.lib()
    return dual_scale_w4a4_amd


def _same(x, y, keys=("a", "b", "codes", "scales", "mse", "g"), name=""):
    for k in keys:
        assert np.array_equal(host(x[k]), host(y[k])), (name, k)


def _layer(scale_down):
    ws = workloads.config5_layer(0, scale_down=scale_down)
    return ws, [to_device(w.W, w.dtype) for w in ws]


@pytest.mark.parametrize("scale_down", [8, 1])
def test_decoder_layer_batch_equals_individual_solves(dq, scale_down):
    ws, Wd = _layer(scale_down)
    w0 = ws[0]
    print(f"[batch] layer 0 /{scale_down}: {[w.W.shape for w in ws]}", flush=True)
    outs = dq.solve_batch(Wd, w0.fmt, w0.group, w0.T)
    for w, W, o in zip(ws, Wd, outs):
        assert o["status"] == 0
        _same(o, dq.solve(W, w.fmt, w.group, w.T), name=w.name)


@pytest.mark.parametrize("per_pass_g", [False, True])
def test_nvfp4_batch(dq, per_pass_g):
    shapes = [(520, 1104), (300, 2048), (96, 512)]
    Ws = [to_device(workloads.config4(r, c).W, "bf16") for r, c in shapes]
    outs = dq.solve_batch(Ws, "nvfp4", 16, 9, per_pass_g=per_pass_g)
    for W, o in zip(Ws, outs):
        _same(o, dq.solve(W, "nvfp4", 16, 9, per_pass_g=per_pass_g))


def test_more_matrices_than_one_launch_takes(dq):
    Ws = [to_device(rand_w(64 + 32 * k, 512 + 64 * (k % 3), seed=k, dtype="bf16"), "bf16")
          for k in range(18)]
    outs = dq.solve_batch(Ws, "int4_bf16", 32, 5)
    for W, o in zip(Ws, outs):
        _same(o, dq.solve(W, "int4_bf16", 32, 5))


def test_mx_batch_equals_the_single_sweep_solves(dq):
    ws = workloads.reduced(3)
    Ws = [to_device(w.W, w.dtype) for w in ws]
    outs = dq.solve_batch(Ws, "mxfp4", 32, 12)
    for W, o in zip(Ws, outs):
        ref = dq.solve(W, "mxfp4", 32, 12, timing=True)
        assert ref["used_fused"]
        _same(o, ref, keys=("a", "b", "codes", "scales"))
        mb, mr = host(o["mse"]), host(ref["mse"])
        assert np.all(np.abs(mb - mr) <= 1e-6 * mr)


def test_batch_error_status(dq):
    good = rand_w(64, 512, seed=1, dtype="bf16")
    bad = good.copy()
    bad[3, 7] = 0x7FC0  # a bf16 NaN
    with pytest.raises(dq.DQError) as e:
        dq.solve_batch([to_device(good, "bf16"), to_device(bad, "bf16")], "mxfp4", 32, 2)
    assert e.value.status == 3

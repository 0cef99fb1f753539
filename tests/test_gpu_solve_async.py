"""GPU tests of the asynchronous solve (dq_solve_async): it enqueues exactly the work of
dq_solve, so its outputs must be bit-identical to the blocking call's (which the solver
parity tests hold to the oracle); several solves may run on several streams with one shared
status word; device errors arrive as status bits; and where the MX single-sweep pass cannot
guarantee its result the call reports it (bit 8) instead of redoing the solve, and the
two-sweep redo gives the blocking call's result."""
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


KEYS = ("codes", "scales", "a", "b", "mse", "g")


def _same(x, y, name):
    for k in KEYS:
        assert np.array_equal(host(x[k]), host(y[k]), equal_nan=True), (name, k)


@pytest.mark.parametrize("fmt,group", [("int4_bf16", 64), ("mxint4", 32), ("mxfp4", 32),
                                       ("nvfp4", 16)])
def test_async_equals_blocking(dq, fmt, group):
    import torch

    W = rand_w(96, 1088, seed=group, outliers=4)  # a ragged column tile
    Wd = to_device(W, "f32")
    print(f"[async] {fmt} G={group}", flush=True)
    want = dq.solve(Wd, fmt, group, 7)
    out = dq.solve_outputs(Wd, fmt, group, 7)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.solve_async(Wd, fmt, group, 7, out, status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 0
    _same(out, want, fmt)


def test_async_on_two_streams_with_one_status(dq):
    import torch

    mats = workloads.reduced(3)  # the MLP pair, reduced
    dev = [to_device(w.W, w.dtype) for w in mats]
    wants = [dq.solve(d, w.fmt, w.group, w.T) for d, w in zip(dev, mats)]
    streams = [torch.cuda.Stream() for _ in mats]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = [dq.solve_outputs(d, w.fmt, w.group, w.T) for d, w in zip(dev, mats)]
    print("[async] two streams, three rounds", flush=True)
    torch.cuda.synchronize()
    for _ in range(3):  # back to back, no wait in between
        for d, w, o, s in zip(dev, mats, outs, streams):
            dq.solve_async(d, w.fmt, w.group, w.T, o, status, stream=s)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 0
    for o, want, w in zip(outs, wants, mats):
        _same(o, want, w.name)


def test_async_status_bits(dq):
    import torch

    W = rand_w(32, 256, seed=7)
    W[3, 17] = np.nan
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    Wd = to_device(W, "f32")
    print("[async] NaN in W", flush=True)
    out = dq.solve_outputs(Wd, "int4_bf16", 32, 3)
    dq.solve_async(Wd, "int4_bf16", 32, 3, out, status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) & 1
    with pytest.raises(dq.DQError) as e:
        dq.solve(Wd, "int4_bf16", 32, 3)
    assert e.value.status == 3


def test_async_reports_the_single_sweep_limit(dq):
    import torch

    # groups scaled far down: the single-sweep identity is not guaranteed there
    W = rand_w(64, 512, seed=4)
    W[5, 64:96] *= np.float32(2.0 ** -118)
    W[9, :32] *= np.float32(2.0 ** -140)
    Wd = to_device(W, "f32")
    print("[async] single-sweep limit", flush=True)
    want = dq.solve(Wd, "mxfp4", 32, 6)  # redoes the solve by itself
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dq.solve_outputs(Wd, "mxfp4", 32, 6)
    dq.solve_async(Wd, "mxfp4", 32, 6, out, status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 8
    status.zero_()
    dq.solve_async(Wd, "mxfp4", 32, 6, out, status, two_sweep=True)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 0
    _same(out, want, "two-sweep redo")

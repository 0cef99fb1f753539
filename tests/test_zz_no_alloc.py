"""GPU test of dq_solve_async_noalloc, the entry point for callers that cannot allocate: its
results must equal those of dq_solve_async with a caller workspace (same kernels, same launch
shape, so bit for bit) on two calls in a row, the second on a smaller matrix, so that the
library's scratch still holds the first call's contents when the second starts. The
reference workspace is filled with garbage first: neither path may expect contents on entry."""
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


def _garbage_workspace(dq, rows, cols, fmt, group):
    import torch

    n = dq.workspace_bytes(rows, cols, fmt, group)
    return torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")


def _pair(dq, W, fmt, group, T, **kw):
    import torch

    rows, cols = W.shape
    print(f"[noalloc] {fmt} G={group} T={T} {rows}x{cols} {kw}", flush=True)
    st_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_new = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = dq.solve_outputs(W, fmt, group, T)
    new = dq.solve_outputs(W, fmt, group, T)
    dq.solve_async(W, fmt, group, T, ref, st_ref,
                   workspace=_garbage_workspace(dq, rows, cols, fmt, group), **kw)
    dq.solve_async_noalloc(W, fmt, group, T, new, st_new, **kw)
    torch.cuda.synchronize()
    assert int(host(st_ref)[0]) == 0 and int(host(st_new)[0]) == 0
    for k in ("codes", "scales", "a", "b", "mse", "g"):
        assert np.array_equal(host(ref[k]), host(new[k])), (fmt, k)
    return new


def test_noalloc_solve_equals_the_workspace_solve_twice(dq):
    # a larger matrix first (its partial sums fill more of the scratch), then a smaller one
    big = workloads.config3("up", 2048, 4096)
    _pair(dq, to_device(big.W, "bf16"), "mxfp4", 32, 6)
    small = rand_w(200, 1088, seed=5, dtype="bf16", outliers=5)
    _pair(dq, to_device(small, "bf16"), "int4_bf16", 32, 5)
    # the two-sweep path, NVFP4 with a per-pass tensor scale, and fp32 weights
    nv = workloads.config4(520, 1104)
    _pair(dq, to_device(nv.W, "bf16"), "nvfp4", 16, 4, per_pass_g=True)
    _pair(dq, to_device(rand_w(96, 512, seed=6), "f32"), "mxint4", 32, 3)


def test_noalloc_rejects_shapes_beyond_its_scratch(dq):
    import torch

    rows, cols = 1 << 17, 16384  # its workspace is larger than the library's scratch
    assert dq.workspace_bytes(rows, cols, "nvfp4", 16) > dq.NOALLOC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")  # never read: rejected on the host
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = dq.lib()
    import ctypes

    init = dq._Init(None, None, 0.0, 0)
    p = fake.data_ptr()
    st = L.dq_solve_async_noalloc(p, 1, rows, cols, 3, 16, 2, ctypes.byref(init), p, p, p, p, p,
                                  p, status.data_ptr(), None)
    assert st == 5  # DQ_ERR_WORKSPACE, before anything is enqueued
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 0

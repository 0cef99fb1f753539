"""GPU tests of the batch solve (dq_solve_batch). Every matrix of a batch is checked two ways:
against the oracle, to the solver's parity bar (exact where no projection decision of the
oracle lies within 1e-9 of a boundary), and against an individual dq_solve of it, which it
must equal bit for bit (same kernels, same order of operations, only the launches shared).
Cases: a decoder layer's seven matrices (reduced, and the full-size last layer), NVFP4 with
fixed and per-pass tensor scales on ragged shapes, more matrices than one launch takes, and
(MX formats, where the individual solve takes the single-sweep path) the single-sweep
results."""
import os

import numpy as np
import pytest

import workloads
from cases import rand_w
from parity import assert_parity, compare_solve, host, to_device

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def dq():
    import torch

    assert torch.cuda.is_available()
    import dual_scale_w4a4_amd

    dual_scale_w4a4_amd.lib()
    return dual_scale_w4a4_amd


@pytest.fixture(scope="module")
def par_oracle(oracle_lib):
    oracle_lib.set_threads(THREADS)  # bit-identical to one thread (pinned)
    yield oracle_lib
    oracle_lib.set_threads(1)


def _same(x, y, keys=("a", "b", "codes", "scales", "mse", "g"), name=""):
    for k in keys:
        assert np.array_equal(host(x[k]), host(y[k])), (name, k)


def _against_oracle(oracle, out, W, dtype, fmt, group, T, name, per_pass_g=False):
    """The batch's result for one matrix against the oracle, to the solver's parity bar."""
    rows, cols = W.shape
    if per_pass_g:
        ref = oracle.solve_pass_g(W, dtype, group, T)
        res = compare_solve(out, ref, fmt, rows, cols)
        assert_parity(res, exact=False, name=name)
        assert res["code_diffs"] == 0 and res["a_flips"] == 0 and res["b_flips"] == 0, (name, res)
    else:
        ref = oracle.solve(W, dtype, fmt, group, T, diag=True)
        res = compare_solve(out, ref, fmt, rows, cols)
        exact = T == 0 or float(ref["margin"].min()) > 1e-9
        assert_parity(res, exact=exact, name=name)
    if fmt == "nvfp4":
        assert host(out["g"])[0] == np.float32(ref["g"]), name
    return res


@pytest.mark.parametrize("scale_down", [8, 1])
def test_decoder_layer_batch_equals_individual_solves(dq, par_oracle, scale_down):
    ws = workloads.config5_layer(0, scale_down=scale_down)
    Wd = [to_device(w.W, w.dtype) for w in ws]
    w0 = ws[0]
    print(f"[batch] layer 0 /{scale_down}: {[w.W.shape for w in ws]}", flush=True)
    outs = dq.solve_batch(Wd, w0.fmt, w0.group, w0.T)
    for w, W, o in zip(ws, Wd, outs):
        assert o["status"] == 0
        _same(o, dq.solve(W, w.fmt, w.group, w.T), name=w.name)
        if scale_down > 1:  # the full-size layer 0 is checked against the oracle elsewhere
            _against_oracle(par_oracle, o, w.W, w.dtype, w.fmt, w.group, w.T, w.name)


def test_last_decoder_layer_full_size_against_oracle(dq, par_oracle):
    # layer 31 of the 32-layer sweep: its own weights and outlier channels
    ws = workloads.config5_layer(31)
    w0 = ws[0]
    print(f"[batch] layer 31: {[w.W.shape for w in ws]}", flush=True)
    outs = dq.solve_batch([to_device(w.W, w.dtype) for w in ws], w0.fmt, w0.group, w0.T)
    for w, o in zip(ws, outs):
        assert o["status"] == 0
        res = _against_oracle(par_oracle, o, w.W, w.dtype, w.fmt, w.group, w.T, w.name)
        print(f"[batch] {w.name}: code_diffs {res['code_diffs']} a/b flips "
              f"{res['a_flips']}/{res['b_flips']} mse_rel {res['mse_rel'][-1]:.2e}", flush=True)


@pytest.mark.parametrize("per_pass_g", [False, True])
def test_nvfp4_batch(dq, par_oracle, per_pass_g):
    shapes = [(520, 1104), (300, 2048), (96, 512)]
    ws = [workloads.config4(r, c) for r, c in shapes]
    Ws = [to_device(w.W, "bf16") for w in ws]
    outs = dq.solve_batch(Ws, "nvfp4", 16, 9, per_pass_g=per_pass_g)
    for w, W, o in zip(ws, Ws, outs):
        _same(o, dq.solve(W, "nvfp4", 16, 9, per_pass_g=per_pass_g))
        _against_oracle(par_oracle, o, w.W, "bf16", "nvfp4", 16, 9, f"nvfp4 {w.W.shape}",
                        per_pass_g=per_pass_g)


def test_more_matrices_than_one_launch_takes(dq, par_oracle):
    Wh = [rand_w(64 + 32 * k, 512 + 64 * (k % 3), seed=k, dtype="bf16") for k in range(18)]
    Ws = [to_device(W, "bf16") for W in Wh]
    outs = dq.solve_batch(Ws, "int4_bf16", 32, 5)
    for k, (Wn, W, o) in enumerate(zip(Wh, Ws, outs)):
        _same(o, dq.solve(W, "int4_bf16", 32, 5))
        _against_oracle(par_oracle, o, Wn, "bf16", "int4_bf16", 32, 5, f"matrix {k}")


def test_mx_batch_equals_the_single_sweep_solves(dq, par_oracle):
    ws = workloads.reduced(3)
    Ws = [to_device(w.W, w.dtype) for w in ws]
    outs = dq.solve_batch(Ws, "mxfp4", 32, 12)
    for w, W, o in zip(ws, Ws, outs):
        ref = dq.solve(W, "mxfp4", 32, 12, timing=True)
        assert ref["used_fused"]
        _same(o, ref, keys=("a", "b", "codes", "scales"))
        mb, mr = host(o["mse"]), host(ref["mse"])
        assert np.all(np.abs(mb - mr) <= 1e-6 * mr)
        _against_oracle(par_oracle, o, w.W, w.dtype, "mxfp4", 32, 12, w.name)


def test_batch_error_status(dq):
    good = rand_w(64, 512, seed=1, dtype="bf16")
    bad = good.copy()
    bad[3, 7] = 0x7FC0  # a bf16 NaN
    with pytest.raises(dq.DQError) as e:
        dq.solve_batch([to_device(good, "bf16"), to_device(bad, "bf16")], "mxfp4", 32, 2)
    assert e.value.status == 3

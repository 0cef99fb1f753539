"""GPU parity of the full solver (dq_solve) against the oracle, plus properties that need
no oracle: determinism, resume, the MX single-sweep path against the two-sweep path, zero
slices, the fallback when the single-sweep identity cannot be guaranteed, and every error
status forced from the host."""
import dataclasses
import os

import numpy as np
import pytest

import fmt_brute as fb
import workloads
from cases import rand_w
from parity import assert_parity, compare_solve, host, scales_np, to_device

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


def _run_pair(dq, oracle, w, T=None, exact_if_margin=1e-9, shape=None):
    T = w.T if T is None else T
    print(f"[solve] {w.name} {w.fmt} G={w.group} T={T} {shape or ''}", flush=True)
    ref = oracle.solve(w.W, w.dtype, w.fmt, w.group, T, diag=True)
    gpu = dq.solve(to_device(w.W, w.dtype), w.fmt, w.group, T, shape=shape)
    res = compare_solve(gpu, ref, w.fmt, w.rows, w.cols)
    exact = T == 0 or float(ref["margin"].min()) > exact_if_margin
    assert_parity(res, exact=exact, name=w.name)
    if w.fmt == "nvfp4":
        assert host(gpu["g"])[0] == np.float32(ref["g"])
    return gpu, ref, res


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_reduced_workloads_match_oracle(dq, par_oracle, cfg):
    for w in workloads.reduced(cfg):
        _run_pair(dq, par_oracle, w)


def test_workload2_full_size(dq, par_oracle):
    _run_pair(dq, par_oracle, workloads.config2())


@pytest.mark.parametrize("which", ["up", "down"])
def test_workload3_full_size(dq, par_oracle, which):
    # 8B-shaped MLP matrices, MXFP4, T = 20: the whole trajectory against the oracle
    gpu, ref, res = _run_pair(dq, par_oracle, workloads.config3(which))
    print(f"[solve] {which}: mse[0]/mse[T] = {ref['mse'][0] / ref['mse'][-1]:.3f} {res}", flush=True)


def test_workload4_full_size(dq, par_oracle):
    gpu, ref, res = _run_pair(dq, par_oracle, workloads.config4())
    print(f"[solve] cfg4: {res}", flush=True)


def test_single_sweep_beyond_the_infinity_cache(dq, par_oracle):
    # a bf16 W of 285 MB, larger than the 256 MiB Infinity Cache, on which the single-sweep
    # pass takes its larger launch (about three workgroups per CU): the 70B-shaped matrix's
    # distribution at 17408 rows, MXFP4 G32 and MXINT4 G32, against the oracle
    base = workloads.config4(rows=17408)
    assert base.W.size * 2 > 256 << 20
    for fmt in ("mxfp4", "mxint4"):
        w = dataclasses.replace(base, name=f"cfg4_rows17408_{fmt}", fmt=fmt, group=32, T=4)
        _run_pair(dq, par_oracle, w)


def test_workload5_first_layer_full_size(dq, par_oracle):
    for w in workloads.config5_layer(0):
        _run_pair(dq, par_oracle, w)


@pytest.mark.parametrize("fmt", ["int4_bf16", "mxint4", "mxfp4", "nvfp4"])
def test_deterministic_and_resumable(dq, fmt):
    group = 16 if fmt == "nvfp4" else 32
    W = to_device(rand_w(300, 1568, seed=9, dtype="bf16", outliers=15), "bf16")
    one = dq.solve(W, fmt, group, 9)
    two = dq.solve(W, fmt, group, 9)
    for k in ("a", "b", "codes", "scales", "mse", "g"):
        assert np.array_equal(host(one[k]), host(two[k])), k
    first = dq.solve(W, fmt, group, 4)
    rest = dq.solve(W, fmt, group, 5, a0=first["a"], b0=first["b"], g0=float(host(first["g"])[0]))
    for k in ("a", "b", "codes", "scales"):
        assert np.array_equal(host(rest[k]), host(one[k])), k
    assert np.array_equal(np.concatenate([host(first["mse"])[:4], host(rest["mse"])]),
                          host(one["mse"]))


@pytest.mark.parametrize("fmt", ["mxint4", "mxfp4"])
def test_single_sweep_equals_two_sweep(dq, fmt):
    for w in workloads.reduced(3):
        W = to_device(w.W, w.dtype)
        fused = dq.solve(W, fmt, 32, 12, timing=True)
        general = dq.solve(W, fmt, 32, 12, two_sweep=True, timing=True)
        assert fused["used_fused"] and not general["used_fused"]
        for k in ("a", "b", "codes", "scales"):
            assert np.array_equal(host(fused[k]), host(general[k])), (w.name, k)
        # same errors summed in a different precision order (fp32 lane sums vs fp64)
        mf, mg = host(fused["mse"]), host(general["mse"])
        assert np.all(np.abs(mf - mg) <= 1e-6 * mg), (w.name, mf, mg)


FUSED_AHEAD_CASES = [
    # (rows, cols, format, group): row counts that end inside an 8-row batch and inside a load
    # step, column counts that end inside a 512-column tile, every group size
    (203, 1088, "mxfp4", 32), (77, 2080, "mxint4", 16), (300, 4096, "mxfp4", 64),
    (33, 512, "mxint4", 32), (517, 96, "mxfp4", 32),
]


@pytest.mark.parametrize("rows,cols,fmt,group", FUSED_AHEAD_CASES)
def test_single_sweep_load_distance_keeps_the_results(dq, oracle_lib, rows, cols, fmt, group):
    # the single-sweep pass with its loads three steps ahead instead of one: the same rows in
    # the same order per wave, so every output is bit-identical, and equal to the oracle's
    T = 6
    Wb = rand_w(rows, cols, seed=rows * 3 + cols, dtype="bf16", outliers=max(1, cols // 200))
    W = to_device(Wb, "bf16")
    print(f"[solve] fused ahead {rows}x{cols} {fmt} G{group}", flush=True)
    far = dq.solve(W, fmt, group, T, shape={"fused_ahead": 3}, timing=True)
    near = dq.solve(W, fmt, group, T, shape={"fused_ahead": 1}, timing=True)
    assert far["used_fused"] and near["used_fused"]
    for k in ("a", "b", "codes", "scales", "mse"):
        assert np.array_equal(host(far[k]), host(near[k])), k
    ref = oracle_lib.solve(Wb, "bf16", fmt, group, T, diag=True)
    res = compare_solve(far, ref, fmt, rows, cols)
    assert_parity(res, exact=float(ref["margin"].min()) > 1e-9, name=f"{rows}x{cols} {fmt}")


def test_single_sweep_falls_back_outside_its_range(dq, oracle_lib):
    # a few groups scaled far down: their shared exponent lies outside the range where the
    # single-sweep identity is guaranteed, so the solver must re-run on the two-sweep path
    W = rand_w(64, 512, seed=4)
    W[5, 64:96] *= np.float32(2.0 ** -118)
    W[9, :32] *= np.float32(2.0 ** -140)
    w = workloads.Workload("extreme", W.astype(np.float32), "f32", "mxfp4", 32, 6)
    gpu = dq.solve(to_device(w.W, "f32"), "mxfp4", 32, 6, timing=True)
    assert not gpu["used_fused"]
    ref = oracle_lib.solve(w.W, "f32", "mxfp4", 32, 6)
    assert_parity(compare_solve(gpu, ref, "mxfp4", 64, 512), exact=True, name="extreme")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxint4"])
def test_single_sweep_row_whose_scaled_values_underflow(dq, oracle_lib, fmt):
    # Row 7 holds bf16 subnormals of at most 3 * 2^-133, so while b >= 2^20 (it starts at
    # 2^22 and moves at most two steps in these iterations) every y = fl32(W rb) of that
    # row rounds to 0 and all its codes are 0 (scale 1 for the slice), although its sum of
    # squares is not 0. The other rows' group maxima stay inside the single-sweep range, so
    # the fast path must keep the solve (no fallback) and give that row a = 1 from 4.
    rows, cols, T = 64, 512, 4
    Wb = rand_w(rows, cols, seed=23, dtype="bf16")
    rng = np.random.default_rng(24)
    Wb[7] = (rng.integers(1, 4, cols) | (rng.integers(0, 2, cols) << 15)).astype(np.uint16)
    a0 = np.ones(rows, np.float32)
    a0[7] = 4.0
    b0 = np.full(cols, 2.0 ** 22, np.float32)
    print(f"[solve] underflow row {fmt}", flush=True)
    gpu = dq.solve(to_device(Wb, "bf16"), fmt, 32, T, a0=a0, b0=b0, timing=True)
    assert gpu["used_fused"]
    two = dq.solve(to_device(Wb, "bf16"), fmt, 32, T, a0=a0, b0=b0, two_sweep=True)
    for k in ("a", "b", "codes", "scales"):
        assert np.array_equal(host(gpu[k]), host(two[k])), k
    ref = oracle_lib.solve(Wb, "bf16", fmt, 32, T, a0=a0, b0=b0, diag=True)
    exact = float(ref["margin"].min()) > 1e-9
    assert_parity(compare_solve(gpu, ref, fmt, rows, cols), exact=exact, name=fmt)
    assert host(gpu["a"])[7] == 1.0
    assert not np.any(fb.unpack_codes(host(gpu["codes"]), fmt)[7])


def test_zero_slices(dq, oracle_lib):
    for fmt in ("int4_bf16", "mxfp4", "nvfp4"):
        group = 16
        W = rand_w(40, 1040, seed=12)
        W[3, :] = 0
        W[:, 17] = 0
        W[8, 32:48] = 0
        gpu = dq.solve(to_device(W, "f32"), fmt, group, 5)
        ref = oracle_lib.solve(W, "f32", fmt, group, 5)
        assert_parity(compare_solve(gpu, ref, fmt, 40, 1040), exact=True, name=fmt)
        assert host(gpu["a"])[3] == 1.0 and host(gpu["b"])[17] == 1.0
        s = fb.decode_scales(scales_np(gpu["scales"], fmt), fmt)
        assert np.all(s[3] == 1.0) and s[8, 2] == 1.0


def test_on_grid_weight_is_a_fixed_point(dq):
    rng = np.random.default_rng(61)
    q = rng.integers(-7, 8, (64, 1024)).astype(np.float64)
    q[:, ::32] = 7.0
    s = fb.bf16_decode(rng.integers(0x3B00, 0x3D00, (64, 32)).astype(np.uint16)).astype(np.float64)
    W = (q * np.repeat(s, 32, axis=1)).astype(np.float32)
    out = dq.solve(to_device(W, "f32"), "int4_bf16", 32, 5)
    assert np.all(host(out["a"]) == 1.0) and np.all(host(out["b"]) == 1.0)
    mse = host(out["mse"])
    assert np.all(mse <= 1e-14 * np.mean(W.astype(np.float64) ** 2))


def test_error_statuses(dq):
    import torch

    W = rand_w(64, 512, seed=2)
    bad = W.copy()
    bad[7, 100] = np.inf
    with pytest.raises(dq.DQError) as e:
        dq.solve(to_device(bad, "f32"), "mxfp4", 32, 3)
    assert e.value.status == 3
    bad[7, 100] = np.nan
    with pytest.raises(dq.DQError) as e:
        dq.quantize(to_device(bad, "f32"), "nvfp4", 16)
    assert e.value.status == 3
    with pytest.raises(dq.DQError) as e:  # scaled tile overflows
        dq.solve(to_device(W * np.float32(1e30), "f32"), "int4_bf16", 32, 2,
                 b0=np.full(512, 1e-30, np.float32))
    assert e.value.status == 4
    with pytest.raises(dq.DQError) as e:  # non-positive init value
        a0 = np.ones(64, np.float32)
        a0[3] = -1
        dq.solve(to_device(W, "f32"), "int4_bf16", 32, 2, a0=a0)
    assert e.value.status == 1
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dq.DQError) as e:
        dq.solve(to_device(W, "f32"), "mxfp4", 32, 2, workspace=ws)
    assert e.value.status == 5
    # a caller-provided workspace of the right size works and matches the allocating call
    ws = torch.empty(dq.workspace_bytes(64, 512, "mxfp4", 32), dtype=torch.uint8, device="cuda")
    x = dq.solve(to_device(W, "f32"), "mxfp4", 32, 3, workspace=ws)
    y = dq.solve(to_device(W, "f32"), "mxfp4", 32, 3)
    assert np.array_equal(host(x["codes"]), host(y["codes"]))


@pytest.mark.parametrize("fmt,two_sweep", [("mxfp4", False), ("mxint4", False),
                                           ("int4_bf16", False), ("mxfp4", True)])
def test_first_pass_row_statistics(dq, oracle_lib, fmt, two_sweep):
    """For bf16 W (T >= 1) the first iteration's pass also forms E_i = sum_j W_ij^2 and the
    finite check, on the single-sweep path and in the two-sweep path's first row pass: a NaN
    or an infinity anywhere in W is reported as non-finite, by the blocking call and in the
    asynchronous status word (bit 1); T = 0 solves (no iteration pass) keep the separate
    row-statistics sweep and match the oracle."""
    import torch

    W = rand_w(96, 1536, seed=31, dtype="bf16", outliers=3)  # bf16 bits
    for bits, where in ((0x7F80, (5, 700)), (0x7FC1, (95, 1535)), (0xFF80, (0, 0))):
        bad = W.copy()
        bad[where] = bits  # +inf, a NaN, -inf
        print(f"[solve] {fmt} bf16 with {bits:#06x} at {where}", flush=True)
        Wd = to_device(bad, "bf16")
        with pytest.raises(dq.DQError) as e:
            dq.solve(Wd, fmt, 32, 4, two_sweep=two_sweep)
        assert e.value.status == 3
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = dq.solve_outputs(Wd, fmt, 32, 4)
        dq.solve_async(Wd, fmt, 32, 4, out, status, two_sweep=two_sweep)
        torch.cuda.synchronize()
        assert int(host(status)[0]) & 1
    # T = 0: setup and emit only; T = 3: the first pass's E_i in every mse[t]
    for T in (0, 3):
        ref = oracle_lib.solve(W, "bf16", fmt, 32, T, diag=True)
        gpu = dq.solve(to_device(W, "bf16"), fmt, 32, T, two_sweep=two_sweep)
        assert_parity(compare_solve(gpu, ref, fmt, 96, 1536),
                      exact=T == 0 or float(ref["margin"].min()) > 1e-9, name=f"{fmt} T={T}")


FIRST_PASS_CASES = [
    # (rows, cols, format, group, T, two_sweep): the two-sweep path's first row pass, which
    # also forms E_i, on ragged shapes (rows ending inside a load step and an 8-row batch,
    # columns ending inside a 1024-column tile, a single row, a 16-column matrix), every group
    # size, T = 1 (that pass and the final one only) and a little more; the MX formats on
    # their two-sweep path
    (203, 1088, "int4_bf16", 32, 1, False), (77, 2112, "int4_bf16", 64, 2, False),
    (1, 512, "int4_bf16", 16, 1, False), (517, 16, "int4_bf16", 16, 3, False),
    (300, 4096, "mxint4", 32, 1, True), (64, 96, "mxfp4", 32, 2, True),
]


@pytest.mark.parametrize("rows,cols,fmt,group,T,two_sweep", FIRST_PASS_CASES)
def test_two_sweep_first_pass_statistics_on_ragged_shapes(dq, oracle_lib, rows, cols, fmt, group,
                                                            T, two_sweep):
    Wb = rand_w(rows, cols, seed=7 * rows + cols, dtype="bf16", outliers=max(1, cols // 200))
    print(f"[solve] first pass {rows}x{cols} {fmt} G{group} T={T}", flush=True)
    gpu = dq.solve(to_device(Wb, "bf16"), fmt, group, T, two_sweep=two_sweep)
    ref = oracle_lib.solve(Wb, "bf16", fmt, group, T, diag=True)
    res = compare_solve(gpu, ref, fmt, rows, cols)
    assert_parity(res, exact=float(ref["margin"].min()) > 1e-9, name=f"{rows}x{cols} {fmt}")


@pytest.mark.parametrize("row_resident", [1, -1])
@pytest.mark.parametrize("fmt", ["int4_bf16", "nvfp4"])
def test_subnormal_groups_on_the_bf16_passes(dq, oracle_lib, fmt, row_resident):
    # bf16 weights with groups of subnormal values: their INT4 scale is a subnormal bf16
    # value, where the codes need the clamp to [-8, 7]; on the row-resident pass and on the
    # two-sweep passes
    group = 16 if fmt == "nvfp4" else 32
    W32 = rand_w(48, 1088, seed=17)
    W32[5, :32] = (np.linspace(-1, 1, 32) * 2.2e-39).astype(np.float32)
    W32[11, 64:96] = (np.linspace(-1, 1, 32) * 5e-40).astype(np.float32)
    Wb = workloads.fp32_to_bf16_bits(W32)
    w = workloads.Workload("subnormal", Wb, "bf16", fmt, group, 4)
    _run_pair(dq, oracle_lib, w, shape={"row_resident": row_resident})


ROW_RESIDENT_CASES = [
    # (rows, cols, format, group, T): ragged row counts (not a multiple of the 8-row batch or
    # of the rows per workgroup), column counts below, at and between whole 512-column waves,
    # every group size, and the widest rows the pass takes
    (203, 1088, "int4_bf16", 32, 7), (77, 2080, "nvfp4", 16, 6), (40, 3072, "int4_bf16", 16, 5),
    (300, 4096, "int4_bf16", 64, 6), (129, 4096, "nvfp4", 16, 5), (1, 512, "int4_bf16", 64, 4),
    (517, 16, "nvfp4", 16, 5), (64, 96, "int4_bf16", 32, 5),
]


@pytest.mark.parametrize("rows,cols,fmt,group,T", ROW_RESIDENT_CASES)
def test_row_resident_pass_equals_two_sweep_and_oracle(dq, oracle_lib, rows, cols, fmt, group, T):
    # the row-resident pass does both Q evaluations of an iteration from one read of each row:
    # the same codes and the same exact products as the two-sweep passes, summed in another
    # fixed fp64 order
    Wb = rand_w(rows, cols, seed=rows + cols, dtype="bf16", outliers=max(1, cols // 200))
    W = to_device(Wb, "bf16")
    rr = dq.solve(W, fmt, group, T, shape={"row_resident": 1}, timing=True)
    assert rr["timing"]["rowres"][1] == T  # one launch per iteration
    two = dq.solve(W, fmt, group, T, shape={"row_resident": -1}, timing=True)
    assert two["timing"]["rowres"][1] == 0
    for k in ("a", "b", "codes", "scales", "g"):
        assert np.array_equal(host(rr[k]), host(two[k])), k
    mr, mt = host(rr["mse"]), host(two["mse"])
    assert np.all(np.abs(mr - mt) <= 1e-12 * mt), (mr, mt)
    ref = oracle_lib.solve(Wb, "bf16", fmt, group, T, diag=True)
    res = compare_solve(rr, ref, fmt, rows, cols)
    assert_parity(res, exact=float(ref["margin"].min()) > 1e-9, name=f"{rows}x{cols} {fmt}")


@pytest.mark.parametrize("shape,T,dtype", [((520, 1104), 20, "bf16"), ((96, 512), 6, "f32"),
                                           ((4096, 8192), 8, "bf16")])
def test_nvfp4_per_pass_tensor_scale(dq, par_oracle, shape, T, dtype):
    # the tensor scale recomputed from each scaled tile before every Q pass
    rows, cols = shape
    w = workloads.config4(rows, cols)
    W = w.W if dtype == "bf16" else workloads.bf16_bits_to_fp32(w.W)
    print(f"[solve] per-pass g {shape} {dtype} T={T}", flush=True)
    ref = par_oracle.solve_pass_g(W, dtype, 16, T)
    gpu = dq.solve(to_device(W, dtype), "nvfp4", 16, T, per_pass_g=True)
    res = compare_solve(gpu, ref, "nvfp4", rows, cols)
    assert_parity(res, exact=False, name=f"per-pass g {shape}")
    assert res["code_diffs"] == 0 and res["a_flips"] == 0 and res["b_flips"] == 0, res
    assert host(gpu["g"])[0] == np.float32(ref["g"])


def test_per_pass_tensor_scale_rejects_a_fixed_one(dq):
    W = to_device(rand_w(64, 512, seed=2), "f32")
    with pytest.raises(dq.DQError) as e:
        dq.solve(W, "nvfp4", 16, 2, g0=0.01, per_pass_g=True)
    assert e.value.status == 1


def _nvfp4_tie_rows(rows, cols, seed):
    """bf16 weights whose first NVFP4 pass meets exact E2M1 ties: the largest element is
    2688 * 2^-10, so g = 2^-10 exactly, and every third row has groups whose maximum is 6 s0 g
    (inner scale s0 = 1 or 1.5, d = s0 g) with the other elements on the decision points
    (1/4, 3/4, ..., 5) times d."""
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.003, (rows, cols)).astype(np.float32)
    W[0, 0] = np.float32(2688 * 2.0 ** -10)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for i in range(1, rows, 3):
        d = (1.0 if i % 2 else 1.5) * 2.0 ** -10
        for c0 in range(16 * (i % 4), cols - 15, 64):
            ks = rng.choice(mids, 16) * rng.choice([-1.0, 1.0], 16)
            ks[rng.integers(16)] = 6.0
            W[i, c0:c0 + 16] = (ks * d).astype(np.float32)
    return workloads.fp32_to_bf16_bits(W)


@pytest.mark.parametrize("rows,cols,per_pass_g", [(96, 1024, False), (301, 2080, False),
                                                  (160, 1104, True)])
def test_nvfp4_ties_in_the_iteration_passes(dq, oracle_lib, rows, cols, per_pass_g):
    # bf16 weights and E4M3 scales make exact E2M1 ties common in NVFP4's two-sweep passes
    # (here planted in the first pass): the codes must settle them to the even index, as the
    # oracle's exact quotient does
    T = 5
    Wb = _nvfp4_tie_rows(rows, cols, seed=rows + cols)
    print(f"[solve] nvfp4 ties {rows}x{cols} per_pass_g={per_pass_g}", flush=True)
    gpu = dq.solve(to_device(Wb, "bf16"), "nvfp4", 16, T, per_pass_g=per_pass_g)
    if per_pass_g:
        ref = oracle_lib.solve_pass_g(Wb, "bf16", 16, T)
        res = compare_solve(gpu, ref, "nvfp4", rows, cols)
        assert_parity(res, exact=False, name=f"ties per-pass g {rows}x{cols}")
        assert res["code_diffs"] == 0 and res["a_flips"] == 0 and res["b_flips"] == 0, res
    else:
        ref = oracle_lib.solve(Wb, "bf16", "nvfp4", 16, T, diag=True)
        assert host(gpu["g"])[0] == np.float32(2.0 ** -10) == np.float32(ref["g"])
        res = compare_solve(gpu, ref, "nvfp4", rows, cols)
        assert_parity(res, exact=float(ref["margin"].min()) > 1e-9, name=f"ties {rows}x{cols}")

"""CPU-side checks of the C ABI: the library loads, exports every entry point the header
declares, and rejects invalid arguments on the host before touching the GPU."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dq.h")
BENCH_HEADER = os.path.join(ROOT, "include", "dq_bench.h")


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def dqlib():
    import dual_scale_w4a4_amd as dq

    if not os.path.exists(dq.LIB_PATH):
        from dual_scale_w4a4_amd import build

        build.build()
    return dq


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == ["dq_act_workspace_bytes", "dq_batch_workspace_bytes", "dq_gemm_mx",
                     "dq_gemm_mx_packed", "dq_gemm_pack_bytes", "dq_gemm_pack_weights",
                     "dq_quantize", "dq_quantize_act", "dq_quantize_act_async", "dq_solve",
                     "dq_solve_async", "dq_solve_async_noalloc", "dq_solve_batch",
                     "dq_status_str", "dq_workspace_bytes"]


def test_bench_header_declares_only_the_measurement_hooks():
    assert _declared_functions(BENCH_HEADER) == ["dq_bench_fp4_mfma_rate",
                                                 "dq_bench_workspace_bytes", "dq_solve_timed"]
    # the solver's own header carries no timing or launch-shape types
    src = open(HEADER).read()
    assert "dq_timing" not in src and "launch_shape" not in src


def test_library_exports_every_declared_symbol(dqlib):
    lib = dqlib.lib()
    declared = _declared_functions() + _declared_functions(BENCH_HEADER)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dqlib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(declared) <= exported


def test_library_is_built_for_gfx950(dqlib):
    out = subprocess.run(["strings", dqlib.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out


def test_status_strings(dqlib):
    for code, name in dqlib.STATUS.items():
        assert dqlib.status_str(code).startswith(name)


def test_workspace_bytes_validates_shape(dqlib):
    assert dqlib.workspace_bytes(128, 256, "int4_bf16", 32) > 0
    assert dqlib.workspace_bytes(128, 250, "int4_bf16", 32) == 0  # cols % group
    assert dqlib.workspace_bytes(128, 256, "int4_bf16", 48) == 0  # group
    assert dqlib.workspace_bytes(0, 256, "mxfp4", 32) == 0
    big = dqlib.workspace_bytes(14336, 4096, "mxfp4", 32)
    assert 0 < big < 64 << 20  # partial sums stay a few percent of W


def test_invalid_arguments_are_rejected_on_the_host(dqlib):
    L = dqlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail first
    init = dqlib._Init(None, None, 0.0, 0)
    args = dict(W=fake, wt=1, rows=128, cols=256, fmt=2, group=32, T=4)

    def call(**kw):
        a = dict(args, **kw)
        return L.dq_solve(a["W"], a["wt"], a["rows"], a["cols"], a["fmt"], a["group"], a["T"],
                          ctypes.byref(init), fake, fake, fake, fake, fake, fake, None, 0, None)

    assert call(W=None) == 1
    assert call(rows=0) == 1
    assert call(cols=250) == 1
    assert call(group=8) == 1
    assert call(T=-1) == 1
    assert call(fmt=9) == 2
    assert call(wt=5) == 2
    assert call(W=ctypes.c_void_p(0x1004)) == 1  # W not 16-byte aligned
    # workspace too small: rejected before any launch
    st = L.dq_solve(fake, 1, 128, 256, 2, 32, 4, ctypes.byref(init), fake, fake, fake, fake,
                    fake, fake, fake, 16, None)
    assert st == 5
    st = L.dq_quantize(fake, 1, 128, 256, 3, 32, None, None, None, fake, fake, None, 0, None)
    assert st == 1  # NVFP4 needs the tensor-scale pointer
    # b is read in 128-bit loads, a as floats
    for a_ptr, b_ptr in ((fake, ctypes.c_void_p(0x1004)), (ctypes.c_void_p(0x1002), fake)):
        st = L.dq_solve(fake, 1, 128, 256, 2, 32, 4, ctypes.byref(init), fake, fake, fake, a_ptr,
                        b_ptr, fake, None, 0, None)
        assert st == 1

    # the asynchronous solve checks the same, and its status pointer
    def call_async(status=fake, init_=init, **kw):
        a = dict(args, **kw)
        return L.dq_solve_async(a["W"], a["wt"], a["rows"], a["cols"], a["fmt"], a["group"],
                                a["T"], ctypes.byref(init_), fake, fake, fake, fake, fake, fake,
                                status, None, 0, None)

    assert call_async(W=None) == 1
    assert call_async(cols=250) == 1
    assert call_async(fmt=9) == 2
    assert call_async(status=None) == 1
    assert call_async(status=ctypes.c_void_p(0x1002)) == 1

    # the allocation-free solve: the same checks, then shapes beyond its scratch, all on the
    # host before any HIP call
    def call_noalloc(status=fake, **kw):
        a = dict(args, **kw)
        return L.dq_solve_async_noalloc(a["W"], a["wt"], a["rows"], a["cols"], a["fmt"],
                                        a["group"], a["T"], ctypes.byref(init), fake, fake, fake,
                                        fake, fake, fake, status, None)

    assert call_noalloc(W=None) == 1
    assert call_noalloc(cols=250) == 1
    assert call_noalloc(status=None) == 1
    assert dqlib.workspace_bytes(1 << 17, 16384, "nvfp4", 16) > dqlib.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(rows=1 << 17, cols=16384, fmt=3, group=16) == 5

    # the measurement entry point: the same checks, and launch-shape fields in range
    def call_timed(shape=None, **kw):
        a = dict(args, **kw)
        return L.dq_solve_timed(a["W"], a["wt"], a["rows"], a["cols"], a["fmt"], a["group"],
                                a["T"], ctypes.byref(init), fake, fake, fake, fake, fake, fake,
                                None, 0, ctypes.byref(shape) if shape else None, None, None)

    assert call_timed(W=None) == 1
    assert call_timed(fmt=9) == 2
    assert call_timed(shape=dqlib._Shape(3, 0, 0, 0, 0)) == 1  # halves: 1 or 2
    assert call_timed(shape=dqlib._Shape(0, 3, 0, 0, 0)) == 1  # step rows: 2 or 4
    assert call_timed(shape=dqlib._Shape(0, 0, 70000, 0, 0)) == 1
    assert call_timed(shape=dqlib._Shape(fused_ahead=2)) == 1  # steps in flight: 1 or 3
    assert call_timed(shape=dqlib._Shape(fused_ahead=3, fused_step_rows=4)) == 1
    assert call_timed(shape=dqlib._Shape(fused_ahead=3, fused_halves=2)) == 1

    # the matrix-core rate hook checks its arguments before any HIP call
    rate = ctypes.c_double(0.0)
    assert L.dq_bench_fp4_mfma_rate(0, None, ctypes.byref(rate)) == 1
    assert L.dq_bench_fp4_mfma_rate((1 << 20) + 1, None, ctypes.byref(rate)) == 1
    assert L.dq_bench_fp4_mfma_rate(100, None, None) == 1


def test_workspace_size_does_not_depend_on_the_environment(dqlib):
    # the launch shape of the product entry points is fixed: tuning variables in the
    # environment (read by earlier versions) change neither the workspace nor the sums' order
    shapes = [(14336, 4096, "mxfp4", 32), (4096, 14336, "int4_bf16", 64), (300, 1568, "nvfp4", 16),
              (128, 256, "int4_bf16", 32)]
    code = ("import sys, json; sys.path.insert(0, %r); import dual_scale_w4a4_amd as dq; "
            "print(json.dumps([dq.workspace_bytes(*s) for s in %r]))" % (ROOT, shapes))
    env = dict(os.environ, DQ_FUSED_SHAPE="2,4,2048", DQ_PASS_TARGET="3000", DQ_TARGET_WGS="64")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         check=True).stdout
    assert json.loads(out) == [dqlib.workspace_bytes(*s) for s in shapes]
    # the measurement entry point's default shape is the product's; another one differs
    for s in shapes:
        assert dqlib.bench_workspace_bytes(*s) == dqlib.workspace_bytes(*s)
    assert dqlib.bench_workspace_bytes(14336, 4096, "mxfp4", 32, {"fused_target": 2048}) != \
        dqlib.workspace_bytes(14336, 4096, "mxfp4", 32)


def test_act_arguments_are_rejected_on_the_host(dqlib):
    L = dqlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail first
    args = dict(X=fake, xt=1, tokens=64, cols=256, fmt=2, group=32, b=None, g=0.0, codes=fake)

    def call(**kw):
        a = dict(args, **kw)
        return L.dq_quantize_act(a["X"], a["xt"], a["tokens"], a["cols"], a["fmt"], a["group"],
                                 a["b"], a["g"], fake, a["codes"], fake, None, 0, None)

    assert call(X=None) == 1
    assert call(tokens=0) == 1
    assert call(cols=250) == 1
    assert call(group=8) == 1
    assert call(fmt=9) == 2
    assert call(xt=5) == 2
    assert call(X=ctypes.c_void_p(0x1008)) == 1      # X not 16-byte aligned
    assert call(codes=ctypes.c_void_p(0x1004)) == 1  # codes not 8-byte aligned
    assert call(b=ctypes.c_void_p(0x1004)) == 1      # b not 16-byte aligned
    assert call(g=float("nan")) == 1
    assert dqlib.act_workspace_bytes(64, 256, "nvfp4", 16) > 0
    assert dqlib.act_workspace_bytes(64, 250, "nvfp4", 16) == 0

    # the asynchronous variant checks the same, and its status pointer
    def call_async(status=fake, **kw):
        a = dict(args, **kw)
        return L.dq_quantize_act_async(a["X"], a["xt"], a["tokens"], a["cols"], a["fmt"],
                                       a["group"], a["b"], a["g"], fake, a["codes"], fake, status,
                                       None, 0, None)

    assert call_async(X=None) == 1
    assert call_async(cols=250) == 1
    assert call_async(status=None) == 1
    assert call_async(status=ctypes.c_void_p(0x1002)) == 1
    assert call_async(codes=ctypes.c_void_p(0x1004)) == 1


def test_gemm_arguments_are_rejected_on_the_host(dqlib):
    L = dqlib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail first
    args = dict(xc=fake, xs=fake, tokens=64, K=256, wc=fake, ws=fake, a=None, out=128, yt=1,
                Y=fake)

    def call(**kw):
        a = dict(args, **kw)
        return L.dq_gemm_mx(a["xc"], a["xs"], a["tokens"], a["K"], a["wc"], a["ws"], a["a"],
                            a["out"], a["yt"], a["Y"], None)

    assert call(xc=None) == 1
    assert call(ws=None) == 1
    assert call(Y=None) == 1
    assert call(tokens=0) == 1
    assert call(out=0) == 1
    assert call(K=48) == 1                           # not a whole number of 32-blocks
    assert call(K=0) == 1
    assert call(K=2 ** 23) == 1                      # beyond the 32-bit offset budget
    assert call(yt=5) == 2
    assert call(xc=ctypes.c_void_p(0x1008)) == 1     # codes not 16-byte aligned
    assert call(wc=ctypes.c_void_p(0x1004)) == 1
    assert call(a=ctypes.c_void_p(0x1004)) == 1      # a not 16-byte aligned

    # the packed form: K a multiple of 512, sizes, and the same argument checks
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.dq_gemm_pack_bytes(100, 1024, ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert cb.value == 4 * 4 * 4 * 1024 and sb.value == 4 * 4 * 256  # 4 row blocks, 4 stages
    assert L.dq_gemm_pack_bytes(100, 768, ctypes.byref(cb), ctypes.byref(sb)) == 1
    assert L.dq_gemm_pack_bytes(0, 1024, ctypes.byref(cb), ctypes.byref(sb)) == 1
    assert L.dq_gemm_pack_weights(fake, fake, 100, 768, fake, fake, None) == 1
    assert L.dq_gemm_pack_weights(ctypes.c_void_p(0x1008), fake, 100, 1024, fake, fake, None) == 1

    def callp(**kw):
        a = dict(args, **kw)
        return L.dq_gemm_mx_packed(a["xc"], a["xs"], a["tokens"], a["K"], a["wc"], a["ws"],
                                   a["a"], a["out"], a["yt"], a["Y"], None)

    assert callp(K=256) == 1
    assert callp(K=1024, xs=ctypes.c_void_p(0x1008)) == 1   # scales not 16-byte aligned
    assert callp(K=1024, yt=7) == 2
    assert callp(K=1024, Y=None) == 1


def test_batch_arguments_are_rejected_on_the_host(dqlib):
    L = dqlib._batch_lib()
    fake = 0x1000
    item = dqlib._BatchItem(fake, 128, 256, None, None, 0.0, fake, fake, fake, fake, fake, fake)
    items = (dqlib._BatchItem * 1)(item)
    assert L.dq_solve_batch(0, items, 1, 2, 32, 4, 0, None, None, 0, None) == 1  # n
    assert L.dq_solve_batch(1, items, 0, 2, 32, 4, 0, None, None, 0, None) == 2  # fp32 W
    assert L.dq_solve_batch(1, items, 1, 2, 48, 4, 0, None, None, 0, None) == 1  # group
    assert L.dq_solve_batch(1, items, 1, 2, 32, -1, 0, None, None, 0, None) == 1  # T
    bad = (dqlib._BatchItem * 1)(dqlib._BatchItem(fake, 128, 250, None, None, 0.0, fake, fake,
                                                  fake, fake, fake, fake))
    assert L.dq_solve_batch(1, bad, 1, 2, 32, 4, 0, None, None, 0, None) == 1  # cols % group
    assert dqlib.batch_workspace_bytes([(128, 256), (64, 512)], "mxfp4", 32) > 0
    assert dqlib.batch_workspace_bytes([(128, 250)], "mxfp4", 32) == 0

"""Throughput of the dual-scale solver on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is one full dq_solve (setup, T block-coordinate-descent iterations, emit) on every
matrix of the workload, with W already resident in HBM. The default workload is the
Llama-3.1-8B-shaped MLP pair (up 14336x4096 and down 4096x14336, bf16, MXFP4, group 32,
T = 20). `value` is whole-job throughput in weight elements x iterations per second:
sum over matrices of rows*cols*T, divided by the time of a step.

Also reported: the marginal time per iteration from solves with T and T = 1; the dominant
kernel's average duration from HIP events recorded on the solve's stream (a second,
instrumented pass over the same steps) against the HBM roofline; and the CPU oracle timed
on a bounded row sample of the same workload, with the GPU result on that sample checked
against it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
KERNEL_SOURCES = ("dual_scale_w4a4_amd/csrc/dq_kernels.hip", "dual_scale_w4a4_amd/csrc/dq_device.h",
                  "dual_scale_w4a4_amd/csrc/dq_internal.h")
# HBM bytes per launch of the single-sweep MXFP4 kernel on the 8B MLP pair, from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs (KiB per dispatch), each scaled by what the same
# counter reads for an elementwise kernel of known size (fetch reports half of a 512 MiB
# read: x2; write is exact: x1). They hold only for the kernel sources they were taken on.
COUNTERS = {
    "workload": 3,
    "kernel": "k_fused_mx<MXFP4, 32, no emit>",
    "fetch_kib": 57466.9, "fetch_scale": 2.0,  # average over both matrices' launches
    "write_kib": 5968.0, "write_scale": 1.0,
    "sources_sha256": "7658cbac43745f57d0242d226029a0c27ff94d68e64a0d0b8b7b52bc0e001c07",
}
METRIC = "weight elems/s per BCD iteration, % HBM peak; final recon MSE vs oracle"

# The vector-ALU roofline: 256 CUs x 4 SIMDs x 16 lanes issue one VALU lane-instruction each
# per clock at 2.4 GHz (fp32 and fp64 adds, multiplies, fmas and conversions alike; packed
# fp32 is not used), 39.3 * 10^12 lane-instructions/s. VALU lane-instructions per weight
# element of each workload's dominant pass, from rocprofv3 --pmc SQ_INSTS_VALU runs (wave
# instructions per dispatch x 64 / elements, over a step's matrices); valid only for the
# kernel sources they were taken on.
VALU_PEAK = 256 * 4 * 16 * 2.4e9
VALU_SOURCES = KERNEL_SOURCES + ("dual_scale_w4a4_amd/csrc/dq_pass.hip",)
VALU_COUNTERS = {
    "per_elem": {"3/fused": 10.45, "4/row": 19.73, "4/col": 19.45, "5/row": 14.24,
                 "5/col": 14.09},  # workload / pass kind
    "sources_sha256": "dc8264d85ba0c30b7d3a8eef58cc43adcf9968a1bae2e96702fc54638ac3ce92",
}


def _load(workload: int):
    import workloads

    if workload == 3:
        return workloads.full(3), "llama3.1-8b MLP up 14336x4096 + down 4096x14336, bf16, MXFP4 G32, T=20"
    if workload == 4:
        return workloads.full(4), "llama3.1-70b MLP 28672x8192, bf16, NVFP4 G16, T=20"
    if workload == 2:
        return workloads.full(2), "2048x2048 bf16 Student-t, MXINT4 G32, T=15"
    if workload == 1:
        return workloads.full(1), "128x256 fp32 tile, INT4/BF16 G32, T=15"
    if workload == 5:
        return workloads.config5_layer(0), "llama3.1-8b decoder layer 0 (q,k,v,o,gate,up,down), bf16, INT4/BF16 G64, T=15"
    raise SystemExit(f"unknown workload {workload}")


ACT_SOURCES = ("dual_scale_w4a4_amd/csrc/dq_act.hip", "dual_scale_w4a4_amd/csrc/dq_device.h",
               "dual_scale_w4a4_amd/csrc/dq_internal.h")
# HBM bytes of one activation-quantizer step (both 8192-token inputs, MXFP4 G32) from
# rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch, summed over the two dispatches of
# a step), scaled as above; valid only for the sources they were taken on.
ACT_COUNTERS = {
    "fetch_kib": 32899.8 + 114916.3, "fetch_scale": 2.0,
    "write_kib": 17408.0 + 60928.0, "write_scale": 1.0,
    "sources_sha256": "a12db08262690d61829bd69b718dde69dd7d5bdcccce22688031ba01851c2732",
}


def _layer(args):
    import workloads

    layer, only = args
    return workloads.config5_layer(layer, only=only)


def load_layers(layers: int, only=None):
    """The decoder layers 0..layers-1 of workload 5 (seeded, one stream per matrix), drawn by
    a pool of host processes when there are several, with a progress line per layer."""
    if layers <= 1:
        return _layer((0, only))
    from concurrent.futures import ProcessPoolExecutor

    workers = max(1, min(16, os.cpu_count() or 1, layers))
    out = [None] * layers
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=workers) as ex:
        for L, ws in enumerate(ex.map(_layer, [(L, only) for L in range(layers)])):
            out[L] = ws
            print(f"[bench] layer {L} drawn ({time.perf_counter() - t0:.0f} s)", file=sys.stderr,
                  flush=True)
    return [w for ws in out for w in ws]


def sources_sha256(files=KERNEL_SOURCES) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_traffic(workload: int, fused: bool):
    """HBM bytes per launch of the dominant kernel from the stored counter runs, or None when
    they do not apply (another workload, another path, or changed kernel sources)."""
    c = COUNTERS
    if not fused or workload != c["workload"] or sources_sha256() != c["sources_sha256"]:
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0


def settle(run_once, ms: float) -> int:
    """Repeat run_once (one untimed step) until `ms` of wall time have passed and the GPU is
    idle again; returns the number of repeats."""
    import torch

    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        run_once()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def to_device(w_np, dtype: str):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w_np).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w_np)).cuda()


def valu_per_elem(workload: int, kind: str, used_fused: bool, per_pass_g: bool, batch: bool):
    """VALU lane-instructions per element of the dominant pass, where counted on these
    sources (keyed by workload and pass kind)."""
    c = VALU_COUNTERS
    if per_pass_g or batch or sources_sha256(VALU_SOURCES) != c["sources_sha256"]:
        return None
    if kind == "fused" and not used_fused:
        return None
    return c["per_elem"].get(f"{workload}/{kind}")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed repeats of the step for this long before the warm-up steps, "
                         "so that the GPU runs at its steady clock (it takes a few hundred "
                         "milliseconds of work to reach it from idle)")
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sequential", action="store_true",
                    help="solve the matrices of a step one after another on one stream "
                         "(default: each on its own stream, concurrently)")
    ap.add_argument("--only", default="",
                    help="workload 5: solve only these of the layer's matrices (comma list of "
                         "q,k,v,o,gate,up,down), e.g. the small k,v")
    ap.add_argument("--layers", type=int, default=1,
                    help="workload 5: decoder layers per step (layer-by-layer inputs 0..N-1)")
    ap.add_argument("--streams", type=int, default=16,
                    help="concurrent solves: matrix k goes on stream k mod N (at most one "
                         "stream per matrix)")
    ap.add_argument("--oracle-child", default="", help=argparse.SUPPRESS)
    ap.add_argument("--batch", action="store_true",
                    help="solve the step's matrices with one batch solve (shared launches) "
                         "instead of one solve per matrix")
    ap.add_argument("--per-pass-g", action="store_true",
                    help="NVFP4 workloads: recompute the tensor scale before every Q pass")
    ap.add_argument("--gemm", action="store_true",
                    help="time the W4A4 MXFP4 product (dq_gemm_mx) on the Llama-3.1-8B MLP "
                         "up / down shapes at 8192 tokens instead of the solver")
    ap.add_argument("--act", action="store_true",
                    help="measure the activation quantizer instead (x = X b, then Q) on the "
                         "Llama-3.1-8B MLP inputs of 8192 tokens; prints its own JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 512 MiB device-to-device copies (the reference that "
                         "scales HBM byte counters)")
    args = ap.parse_args()
    if args.oracle_child:
        oracle_child(args.oracle_child)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the solver runs each matrix on a single device "
              "(sharding across GPUs is by matrix, with no communication); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # an elementwise kernel that reads 512 MiB and writes 512 MiB
        src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 512 << 20, "copies": args.steps}), flush=True)
        return

    import dual_scale_w4a4_amd as dq

    if args.gemm:
        bench_gemm(args, dq)
        return
    if args.act:
        bench_act(args, dq)
        return

    mats, desc = _load(args.workload)
    if args.workload == 5:
        only = tuple(args.only.split(",")) if args.only else None
        mats = load_layers(args.layers, only)
        desc = desc.replace("layer 0", f"layers 0..{args.layers - 1}" if args.layers > 1 else "layer 0")
        if args.only:
            desc += f", only {args.only}"
    dev_w = [to_device(w.W, w.dtype) for w in mats]
    work = [dq.workspace_bytes(w.rows, w.cols, w.fmt, w.group) for w in mats]
    wss = [torch.empty(b, dtype=torch.uint8, device="cuda") for b in work]
    n_streams = max(1, min(args.streams, len(mats)))
    streams = [torch.cuda.Stream() for _ in range(n_streams)]  # default priority
    torch.cuda.synchronize()
    pool = None
    if not args.sequential and len(mats) > 1:
        from concurrent.futures import ThreadPoolExecutor

        pool = ThreadPoolExecutor(max_workers=n_streams)

    # read in full before each cold re-run of the dominant pass: twice the 256 MB
    # Infinity Cache, so that W is evicted from every cache level
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)

    def solve_one(k, T, timing, stream):
        w = mats[k]
        return dq.solve(dev_w[k], w.fmt, w.group, w.T if T is None else T, workspace=wss[k],
                        timing=timing, stream=stream, flush=flush if timing else None,
                        per_pass_g=args.per_pass_g and w.fmt == "nvfp4")

    batch_ws = None
    if args.batch:
        batch_ws = torch.empty(dq.batch_workspace_bytes([(w.rows, w.cols) for w in mats],
                                                        mats[0].fmt, mats[0].group),
                               dtype=torch.uint8, device="cuda")

    # the timed steps enqueue every solve with dq_solve_async (each matrix on its own stream
    # unless --sequential) and wait once, at the end of the timed region; device errors are
    # OR-ed into one status word, checked after it
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_bufs = {}

    def outs_for(k, T):
        if (k, T) not in out_bufs:
            w = mats[k]
            out_bufs[(k, T)] = dq.solve_outputs(dev_w[k], w.fmt, w.group, T)
        return out_bufs[(k, T)]

    blocking = [False]

    def step(T=None, timing=False):
        if args.batch and not timing:
            w = mats[0]
            return dq.solve_batch(dev_w, w.fmt, w.group, w.T if T is None else T,
                                  per_pass_g=args.per_pass_g and w.fmt == "nvfp4",
                                  workspace=batch_ws)
        if timing or blocking[0]:
            # dq_solve returns when its stream is done; concurrent calls use separate streams
            # and workspaces (the library keeps no global state)
            if pool is None or timing:
                return [solve_one(k, T, timing, None) for k in range(len(mats))]
            # one worker per stream, each solving its own matrices in order
            def worker(j):
                return [(k, solve_one(k, T, False, streams[j]))
                        for k in range(j, len(mats), n_streams)]

            done = dict(kv for f in [pool.submit(worker, j) for j in range(n_streams)]
                        for kv in f.result())
            return [done[k] for k in range(len(mats))]
        res = []
        for k, w in enumerate(mats):
            Tk = w.T if T is None else T
            o = outs_for(k, Tk)
            dq.solve_async(dev_w[k], w.fmt, w.group, Tk, o, status, workspace=wss[k],
                           stream=None if args.sequential else streams[k % n_streams],
                           per_pass_g=args.per_pass_g and w.fmt == "nvfp4")
            res.append(o)
        return res

    settled = [None]

    def timed_steps(T=None):
        if settled[0] is None:
            settled[0] = settle(lambda: step(T), args.settle_ms)
        for _ in range(args.warmup):
            step(T)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            outs = step(T)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps, outs

    t_step, outs = timed_steps()
    if not args.batch and int(status.item()) != 0:
        # a solve needed the two-sweep redo that only the blocking call performs (or failed):
        # time the blocking calls instead, which redo or report it themselves
        blocking[0] = True
        t_step, outs = timed_steps()

    # marginal per-iteration time: solves with T = 1 (setup, one iteration, emit); the first
    # iteration's pass also sums W^2 on the single-sweep path, so T = 1 keeps it on both sides
    t_step1, _ = timed_steps(T=1)

    # instrumented pass over the same steps: per-kernel HIP events on the solve's stream
    bytes_per_elem = 2 if mats[0].dtype == "bf16" else 4
    per_kind, used_fused = {}, True  # kind -> [ms, launches, bytes read by those launches]
    iso = [0.0, 0, 0.0]  # ms, launches, bytes of the isolated back-to-back runs
    cw = [0.0, 0.0, 0, 0.0]  # cold ms, warm ms, launches, bytes of the one-at-a-time re-runs
    for _ in range(args.steps):
        for w, o in zip(mats, step(timing=True)):
            used_fused = used_fused and o["used_fused"]
            for k, (ms, n) in o["timing"].items():
                acc = per_kind.setdefault(k, [0.0, 0, 0.0])
                acc[0] += ms
                acc[1] += n
                acc[2] += n * w.rows * w.cols * bytes_per_elem  # each pass launch reads W once
            iso[0] += o["isolated"][0]
            iso[1] += o["isolated"][1]
            iso[2] += o["isolated"][1] * w.rows * w.cols * bytes_per_elem
            cold, warm, n1 = o["cold_warm"]
            cw[0] += cold
            cw[1] += warm
            cw[2] += n1
            cw[3] += n1 * w.rows * w.cols * bytes_per_elem
    # the dominant kernel: the iteration pass with the most kernel time
    kind = max((k for k in ("fused", "rowres", "row", "col") if per_kind.get(k, [0])[0] > 0),
               key=lambda k: per_kind[k][0])
    ms_kind, n_kind, bytes_total = per_kind[kind]
    if kind == "fused" and iso[1] > 0:  # back-to-back launches between one event pair
        ms_kind, n_kind, bytes_total = iso

    elems = sum(w.rows * w.cols for w in mats)
    elem_iters = sum(w.rows * w.cols * w.T for w in mats)
    T_mean = elem_iters / elems
    value = elem_iters / t_step
    # per iteration over all matrices of the step
    t_iter = (t_step - t_step1) / (T_mean - 1.0) if T_mean > 1.0 else float("nan")
    iter_gbs = elems * bytes_per_elem / t_iter / 1e9
    avg_launch_ms = ms_kind / max(n_kind, 1)
    launch_bytes = bytes_total / max(n_kind, 1)
    achieved = bytes_total / (ms_kind * 1e-3) / 1e9

    kernel_name = {"fused": "k_fused_mx", "rowres": "k_rowres",
                   "row": "k_pass (row mode)" if mats[0].dtype == "bf16" else "k_sweep (row mode)",
                   "col": "k_pass (column mode)" if mats[0].dtype == "bf16" else "k_sweep (column mode)"}[kind]
    roofline = {"bound": "hbm", "kernel": kernel_name, "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": counted_traffic(args.workload, kind == "fused" and used_fused),
                "traffic_unit": "bytes per launch", "avg_launch_us": avg_launch_ms * 1e3,
                "launches": n_kind, "bytes_per_launch": launch_bytes,
                "timing": "isolated back-to-back launches" if (kind == "fused" and iso[1])
                          else "per-launch events, sequential instrumented solves",
                "kernel_share": {k: v[0] / sum(x[0] for x in per_kind.values())
                                 for k, v in per_kind.items() if v[0] > 0}}
    if cw[2] > 0 and kind == "fused":
        # `achieved` above times back-to-back launches, where a matrix that fits the 256 MB
        # Infinity Cache is partly served from it; the cold figure reads W from HBM
        cold_gbs = cw[3] / (cw[0] * 1e-3) / 1e9
        roofline.update({
            "source_of_W": "back-to-back launches: W (<= 256 MB) partly served from the "
                           "Infinity Cache; achieved_cold / frac_cold: one launch after a "
                           "full read of a 512 MiB buffer, W from HBM",
            "achieved_cold": cold_gbs, "frac_cold": cold_gbs / HBM_PEAK_GBS,
            "avg_launch_us_cold": cw[0] / cw[2] * 1e3})
    per_elem = valu_per_elem(args.workload, kind, used_fused, args.per_pass_g, args.batch)
    if per_elem is not None:
        valu = per_elem * (bytes_total / bytes_per_elem) / (ms_kind * 1e-3)
        alu = {"lane_instructions_per_element": per_elem, "achieved": valu / 1e12,
               "peak": VALU_PEAK / 1e12, "unit": "T VALU lane-instructions/s",
               "frac": valu / VALU_PEAK}
        if kind in ("row", "col", "rowres"):  # exact fp64 codes and sums bind the ALU
            hbm = {k: roofline[k] for k in ("achieved", "peak", "unit", "frac")}
            roofline.update(bound="alu", **{k: alu[k] for k in ("achieved", "peak", "unit", "frac")})
            roofline["lane_instructions_per_element"] = per_elem
            roofline["hbm"] = hbm
        else:
            roofline["valu"] = alu

    mse_final = [float(o["mse"][-1].item()) for o in outs]
    mse_first = [float(o["mse"][0].item()) for o in outs]

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "weight-elements x iterations / s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators in workloads/, no checkpoint)",
        "config": {"workload": desc + (", tensor scale per Q pass" if args.per_pass_g else "")
                   + (", one batch solve" if args.batch else ""),
                   "matrices": [w.name for w in mats],
                   "format": mats[0].fmt, "group": mats[0].group, "T": mats[0].T,
                   "weights": mats[0].dtype, "sums": "f64"},
        "settle": {"ms": args.settle_ms, "untimed_steps": settled[0],
                   "why": "the GPU reaches its steady clock only after a few hundred ms of work"},
        "solve_calls": "blocking dq_solve" if (blocking[0] or args.batch) else
                       "dq_solve_async, one wait per timed region",
        "device_status": int(status.item()),
        "per_iteration": {"ms": t_iter * 1e3, "elems_per_s": elems / t_iter,
                          "GBps_one_read_of_W": iter_gbs, "frac_hbm_peak": iter_gbs / HBM_PEAK_GBS,
                          "ms_per_step_T1": t_step1 * 1e3},
        "roofline": roofline,
        "mse": {"first": mse_first, "final": mse_final,
                "ratio_first_over_final": [a / b for a, b in zip(mse_first, mse_final)]},
        "cache": None if cw[2] == 0 else {
            "method": "dominant pass timed one launch at a time with HIP events, cold = after "
                      "a full read of a 512 MiB buffer (evicts W from L2 and the 256 MB "
                      "Infinity Cache), warm = back to back (W of 117 MB can stay in it)",
            "cold_us": cw[0] / cw[2] * 1e3, "warm_us": cw[1] / cw[2] * 1e3,
            "cold_GBps": cw[3] / (cw[0] * 1e-3) / 1e9, "warm_GBps": cw[3] / (cw[1] * 1e-3) / 1e9,
            "warm_over_cold_speed": cw[0] / cw[1]},
        "single_sweep_path": used_fused if kind == "fused" else None,
        "concurrent_matrices": pool is not None and not args.batch,
        "batch_solve": args.batch,
    }

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(mats[0], dq, to_device, args.per_pass_g)
    print(json.dumps(line), flush=True)


def act_traffic():
    c = ACT_COUNTERS
    if sources_sha256(ACT_SOURCES) != c["sources_sha256"]:
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0


def bench_act(args, dq) -> None:
    """The activation quantizer on the Llama-3.1-8B MLP inputs of a batch of 8192 tokens
    (8192 x 4096 into up / gate, 8192 x 14336 into down), bf16, MXFP4 G32 and NVFP4 G16 (g
    given), each a step of both inputs. Kernel time: back-to-back asynchronous calls between
    one pair of HIP events on the calling stream. Algorithmic bytes per element: read X (2 B),
    write the code (0.5 B) and 1/G of an inner-scale byte."""
    import numpy as np
    import torch

    import workloads

    stream = torch.cuda.current_stream()
    inputs = []
    for name in ("up", "down"):
        X, b = workloads.act_inputs(name)
        inputs.append((name, to_device(X, "bf16"), to_device(b, "f32")))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    results = {}
    for fmt, group, g in (("mxfp4", 32, 0.0), ("nvfp4", 16, 0.01)):
        outs = []
        for name, Xd, bd in inputs:
            o = dq.quantize_act(Xd, fmt, group, bd, g=g)
            outs.append((name, Xd, bd, o["codes"], o["scales"]))
        def step():
            for name, Xd, bd, codes, scales in outs:
                dq.quantize_act_async(Xd, fmt, group, codes, scales, status, b=bd, g=g,
                                      stream=stream)
        settled = settle(step, args.settle_ms)
        for _ in range(args.warmup):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        elems = sum(Xd.numel() for _, Xd, _, _, _ in outs)
        algo = elems * (2.0 + 0.5 + 1.0 / group)
        results[fmt] = {"group": group, "ms_per_step": ms, "elems_per_s": elems / (ms * 1e-3),
                        "settle_steps": settled,
                        "achieved_GBps": algo / (ms * 1e-3) / 1e9,
                        "frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "bytes_per_step": algo}
    assert int(status.item()) == 0
    m = results["mxfp4"]
    # the CPU oracle on a bounded sample: the whole 8192-token up input
    import oracle

    Xs, bs = workloads.act_inputs("up")
    Xs = np.ascontiguousarray(Xs)
    t0 = time.perf_counter()
    ref = oracle.quantize_act(Xs, "bf16", "mxfp4", 32, bs)
    dt = time.perf_counter() - t0
    got = dq.quantize_act(to_device(Xs, "bf16"), "mxfp4", 32, to_device(bs, "f32"))
    same = bool(np.array_equal(got["codes"].cpu().numpy(), ref["codes"]) and
                np.array_equal(got["scales"].cpu().numpy(), ref["scales"]))
    line = {
        "metric": "activation quantization (x = X b, then Q) elements/s, % HBM peak",
        "value": m["elems_per_s"], "unit": "activation elements / s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": m["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded generators in workloads/)",
        "config": {"workload": "llama3.1-8b MLP inputs of 8192 tokens: 8192x4096 + 8192x14336, "
                               "bf16, MXFP4 G32 (NVFP4 G16 with a given g alongside)"},
        "roofline": {"bound": "hbm", "kernel": "k_act", "achieved": m["achieved_GBps"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": m["frac"],
                     "traffic": act_traffic(), "traffic_unit": "bytes per step",
                     "timing": "back-to-back asynchronous calls between one pair of events"},
        "formats": results,
        "cpu_baseline": {"value": Xs.size / dt, "unit": "activation elements / s", "cores": 1,
                         "kind": "oracle", "sample": "the whole 8192x4096 input, MXFP4 G32",
                         "seconds": dt, "gpu_identical_on_sample": same},
    }
    print(json.dumps(line), flush=True)


FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix-core peak
GEMM_SOURCES = ("dual_scale_w4a4_amd/csrc/dq_gemm.hip",)
# HBM bytes of one W4A4 step (up and down with packed weights) from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs (KiB per dispatch, summed over the two products), scaled as above; valid
# only for the kernel source they were taken on.
GEMM_COUNTERS = {
    "fetch_kib": 183036.5 + 183980.5, "fetch_scale": 2.0,
    "write_kib": 229431.8 + 65549.1, "write_scale": 1.0,
    "sources_sha256": "7a106e97d909772488dc3e4b27c6650f732a37fc80a822acb09a5428608415d2",
}


def gemm_traffic():
    c = GEMM_COUNTERS
    if sources_sha256(GEMM_SOURCES) != c["sources_sha256"]:
        return None
    return (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0


def bench_gemm(args, dq) -> None:
    """The W4A4 product on the chain it serves: the Llama-3.1-8B MLP up (14336x4096) and down
    (4096x14336) weights solved on the GPU (MXFP4 G32, T = 20) and packed once for the matrix
    cores (dq_gemm_pack_weights: static weights, like the solve itself outside the timed
    region), the MLP inputs of 8192 tokens quantized with the solver's b, and a step = both
    products Y = (xhat Qhat^T) D_a with the packed weights, bf16 out. The same products from
    the weights as the solver writes them (dq_gemm_mx) are timed alongside. Kernel time:
    back-to-back calls between one pair of HIP events on the calling stream. Algorithmic
    flops: 2 * tokens * out * K per product."""
    import numpy as np
    import torch

    import workloads

    stream = torch.cuda.current_stream()
    mats = []
    for w, name in zip(workloads.full(3), ("up", "down")):
        sol = dq.solve(to_device(w.W, w.dtype), "mxfp4", 32, w.T)
        X, b = workloads.act_inputs(name)
        act = dq.quantize_act(to_device(X, "bf16"), "mxfp4", 32, sol["b"])
        del X
        tokens, K = act["codes"].shape[0], act["codes"].shape[1] * 2
        out = sol["codes"].shape[0]
        y = torch.empty((tokens, out), dtype=torch.bfloat16, device="cuda")
        packed = dq.gemm_pack_weights(sol["codes"], sol["scales"])
        mats.append(dict(name=name, xc=act["codes"], xs=act["scales"], wc=sol["codes"],
                         ws=sol["scales"], a=sol["a"], y=y, flops=2.0 * tokens * out * K,
                         shape=(tokens, out, K), packed=packed))

    def run(ms_list, packed):
        for m in ms_list:
            if packed:
                dq.gemm_mx_packed(m["xc"], m["xs"], m["packed"], m["a"], out_dtype="bf16",
                                  y=m["y"], stream=stream)
            else:
                dq.gemm_mx(m["xc"], m["xs"], m["wc"], m["ws"], m["a"], out_dtype="bf16",
                           y=m["y"], stream=stream)

    settled = settle(lambda: run(mats, True), args.settle_ms)

    def timed(ms_list, steps, packed):
        for _ in range(args.warmup):
            run(ms_list, packed)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            run(ms_list, packed)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(mats, args.steps, True)
    ms_natural = timed(mats, args.steps, False)
    flops = sum(m["flops"] for m in mats)
    per = {}
    for m in mats:
        for packed in (True, False):
            t = timed([m], args.steps, packed)
            per[m["name"] + ("" if packed else " (unpacked weights)")] = {
                "shape_tokens_out_k": m["shape"], "ms": t,
                "tflops": m["flops"] / (t * 1e-3) / 1e12,
                "frac": m["flops"] / (t * 1e-3) / 1e12 / FP4_MFMA_PEAK_TFLOPS}
    tf = flops / (ms * 1e-3) / 1e12
    # what the matrix cores sustain on this instruction with nothing but register operands
    attainable = max(dq.bench_fp4_mfma_rate(20000, stream=stream) for _ in range(2))
    line = {
        "metric": "W4A4 MXFP4 product TFLOP/s (dense-equivalent), % FP4 matrix-core peak",
        "value": tf, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp4 (E2M1 x E2M1, E8M0 block scales, fp32 accumulate)",
        "data": "synthetic (seeded generators in workloads/), weights and activations "
                "quantized on the GPU by the solver and the activation quantizer",
        "config": {"workload": "llama3.1-8b MLP at 8192 tokens: up 8192x4096 x (14336x4096)^T "
                               "+ down 8192x14336 x (4096x14336)^T, MXFP4 G32, bf16 out"},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_mx_packed", "achieved": tf,
                     "peak": FP4_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / FP4_MFMA_PEAK_TFLOPS, "traffic": gemm_traffic(),
                     "attainable": attainable, "frac_attainable": tf / attainable,
                     "attainable_note": "the same instruction streamed on register operands "
                                        "alone (dq_bench_fp4_mfma_rate): the chip's clock "
                                        "drops under full matrix-core load",
                     "traffic_unit": "HBM bytes per step",
                     "timing": "back-to-back asynchronous calls between one pair of events"},
        "products": per,
        "unpacked_weights_tflops": flops / (ms_natural * 1e-3) / 1e12,
        "settle": {"ms": args.settle_ms, "untimed_steps": settled},
    }
    if args.no_cpu:
        print(json.dumps(line), flush=True)
        return
    # the CPU oracle on a bounded sample: 256 tokens of the up product, every output channel
    import oracle

    m = mats[0]
    ts = np.arange(256)
    xc, xs = m["xc"][ts].cpu().numpy(), m["xs"][ts].cpu().numpy()
    wc, ws, a = m["wc"].cpu().numpy(), m["ws"].cpu().numpy(), m["a"].cpu().numpy()
    threads = oracle.set_threads(min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    ref = oracle.gemm_mx(xc, xs, wc, ws, a)
    dt = time.perf_counter() - t0
    oracle.set_threads(1)
    run([m], True)
    torch.cuda.synchronize()
    got = m["y"][ts].float().cpu().numpy().astype(np.float64)
    rel = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)))
    sample_flops = 2.0 * len(ts) * wc.shape[0] * xc.shape[1] * 2
    line["cpu_baseline"] = {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s",
                            "cores": threads, "kind": "oracle",
                            "sample": "256 tokens x 14336 channels x K=4096 of the up product",
                            "seconds": dt, "gpu_max_rel_err_on_sample_bf16": rel}
    print(json.dumps(line), flush=True)


def oracle_child(spec: str) -> None:
    """Run in a child process pinned to one core: the oracle, single-threaded, on a sample
    saved by the parent; prints its wall time as JSON."""
    import numpy as np

    import oracle

    d = json.loads(spec)
    sample = np.load(d["path"], allow_pickle=False)
    threads = oracle.set_threads(1)
    t0 = time.perf_counter()
    if d["pass_g"]:
        oracle.solve_pass_g(sample, d["dtype"], d["group"], d["T"])
    else:
        oracle.solve(sample, d["dtype"], d["fmt"], d["group"], d["T"])
    dt = time.perf_counter() - t0
    print(json.dumps({"seconds": dt, "threads": threads, "affinity": sorted(os.sched_getaffinity(0))}))


def cpu_single_core(w, per_pass_g: bool):
    """The oracle on one host core: a child process pinned to one core (taskset -c 0, else
    sched_setaffinity in the child) on rows 0..R-1 of the matrix, R about 4M / cols."""
    import shutil
    import subprocess
    import tempfile

    import numpy as np

    rows = min(w.rows, max(16, (1024 * 4096) // w.cols))
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "sample.npy")
        np.save(path, np.ascontiguousarray(w.W[:rows]))
        spec = json.dumps({"path": path, "dtype": w.dtype, "fmt": w.fmt, "group": w.group,
                           "T": w.T, "pass_g": bool(per_pass_g and w.fmt == "nvfp4")})
        cmd = [sys.executable, os.path.abspath(__file__), "--oracle-child", spec]
        env = dict(os.environ, OMP_NUM_THREADS="1")
        if shutil.which("taskset"):
            cmd, how = ["taskset", "-c", "0"] + cmd, "taskset -c 0"
        else:
            env["DQ_BENCH_PIN_CPU"] = "0"
            how = "sched_setaffinity"
        res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
        if res.returncode != 0:
            return {"error": res.stderr[-500:]}
        d = json.loads(res.stdout.strip().splitlines()[-1])
    return {"value": rows * w.cols * w.T / d["seconds"], "unit": "weight-elements x iterations / s",
            "cores": 1, "pinned": how, "affinity": d["affinity"], "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of {w.name} ({rows}x{w.cols}), {w.fmt}, T={w.T}",
            "seconds": d["seconds"]}


def cpu_baseline(w, dq, to_device, per_pass_g=False):
    """The oracle on a bounded row sample of the first matrix (same T), all host cores up to
    16, and the GPU on the same sample checked against it; beside it the oracle on one pinned
    core, on a smaller sample."""
    import numpy as np

    import oracle

    rows = min(w.rows, max(64, (8192 * 4096) // w.cols))
    sample = np.ascontiguousarray(w.W[:rows])
    threads = oracle.set_threads(min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    pp = per_pass_g and w.fmt == "nvfp4"
    if pp:
        ref = oracle.solve_pass_g(sample, w.dtype, w.group, w.T)
    else:
        ref = oracle.solve(sample, w.dtype, w.fmt, w.group, w.T)
    dt = time.perf_counter() - t0
    oracle.set_threads(1)
    gpu = dq.solve(to_device(sample, w.dtype), w.fmt, w.group, w.T, per_pass_g=pp)
    mse_g = gpu["mse"].cpu().numpy()
    a_eq = bool(np.array_equal(gpu["a"].cpu().numpy(), ref["a"]))
    b_eq = bool(np.array_equal(gpu["b"].cpu().numpy(), ref["b"]))
    codes_eq = bool(np.array_equal(gpu["codes"].cpu().numpy(), ref["codes"]))
    return {
        "value": rows * w.cols * w.T / dt,
        "unit": "weight-elements x iterations / s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of {w.name} ({rows}x{w.cols}), {w.fmt}, T={w.T}",
        "seconds": dt,
        "gpu_vs_oracle_on_sample": {"mse_final_rel": float(abs(mse_g[-1] - ref["mse"][-1]) / ref["mse"][-1]),
                                    "a_identical": a_eq, "b_identical": b_eq,
                                    "codes_identical": codes_eq},
        "single_core": cpu_single_core(w, per_pass_g),
    }


if __name__ == "__main__":
    if os.environ.get("DQ_BENCH_PIN_CPU"):
        os.sched_setaffinity(0, {int(os.environ["DQ_BENCH_PIN_CPU"])})
    main()

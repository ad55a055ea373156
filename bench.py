#!/usr/bin/env python3
"""Benchmark of the FP32 row-reduction library on one MI355X.

One step = one rmsnorm_f32 call (plan lookup, vectorised load, per-lane sum of
squares, wavefront and LDS reduction, rsqrt-scale epilogue and store) over the
bandwidth-bound 16384x8192 RMSNorm workload (x ~ N(0,1), w ~ U(0.5,1.5),
eps = 1e-6), inputs resident in HBM. Prints one JSON line:

  value      whole-job throughput of the timed steps in algorithmic GB/s
             (bytes = 8*rows*cols + 4*cols per call: x read once, y written
             once, w read once)
  roofline   the RMSNorm kernel's achieved GB/s (algorithmic bytes / average
             kernel duration from HIP events on the launch stream) against
             MI355X's 8 TB/s HBM peak; `traffic` from hardware counters when
             a committed counter summary matches the current kernel source
  cpu_baseline  the CPU oracle timed on host cores over a bounded sample
  shapes     per-shape us/op, rows/s, GB/s and fraction of peak for every
             measured RMSNorm shape and the five sibling operators, next to
             an empty-kernel launch floor and a same-bytes copy ceiling
  long_rows  few long rows: one workgroup per row against split rows
  streaming_rows  many rows beyond the register path (vocabulary-size
             cross-entropy and softmax, 65536-column normalisations)
  single_call  end-to-end latency of one tiny call (C entry point and
             binding), and the 24-call operator-coverage set as separate
             launches against one batched launch

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-shapes] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "FP32 RMSNorm µs/op + achieved HBM GB/s (% of MI355X peak) per shape"
HEADLINE = (16384, 8192)
COLD_SET_BYTES = 768 << 20  # distinct buffers cycled for cache-cold timings


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Fingerprint of the RMSNorm kernel as launched here: its device sources
    and the selected plan (the counter summary records the same)."""
    from row_reduction_amd.profile_cases import headline_fingerprint
    return headline_fingerprint()


def counter_traffic(source_hash: str):
    """Bytes per launch from the committed counter summary, if it was taken on
    this exact kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "rmsnorm_16384x8192_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash:
        return None
    return float(t.group(1))


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.start = torch.cuda.Event(enable_timing=True)
        self.stop = torch.cuda.Event(enable_timing=True)

    def time_ms(self, fn, n: int) -> float:
        self.start.record()
        for _ in range(n):
            fn()
        self.stop.record()
        self.stop.synchronize()
        return self.start.elapsed_time(self.stop)


def batch_us(torch, fn, target_ms: float = 20.0, rounds: int = 3, samples: int = 5) -> dict:
    """Median of per-round medians of batch-amortised microseconds per call."""
    timer = Timer(torch)
    fn()
    torch.cuda.synchronize()
    probe = timer.time_ms(fn, 5) / 5
    n = max(5, min(20000, int(target_ms / max(probe, 1e-3))))
    per_round = []
    raw = []
    for _ in range(rounds):
        vals = sorted(timer.time_ms(fn, n) * 1000.0 / n for _ in range(samples))
        raw.extend(vals)
        per_round.append(vals[len(vals) // 2])
    per_round.sort()
    return {"us": per_round[len(per_round) // 2], "min_us": min(raw), "max_us": max(raw),
            "launches_per_sample": n}


def graph_us(torch, fn, n: int, samples: int = 15) -> dict:
    """Median us per call over replays of a HIP graph of n calls of fn."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    timer = Timer(torch)
    g.replay()
    torch.cuda.synchronize()
    vals = sorted(timer.time_ms(g.replay, 1) * 1000.0 / n for _ in range(samples))
    return {"us": vals[len(vals) // 2], "min_us": vals[0], "max_us": vals[-1]}


def shape_table(torch, rr, workloads, device, samples: int = 15) -> list:
    """us/op and GB/s for every measured shape and operator with the selected
    plan. Each sample replays a HIP graph of back-to-back launches (GPU time
    per call, host launch cost excluded); working sets of 1 MiB or more are
    also timed cold, cycling >= 768 MiB of distinct buffers. `single_call_us`
    is one synchronised host call, launch to completion. `copy_same_shape_*`
    is rr_copy_f32 over a matrix of the same shape and element size timed the
    same way: the practical per-call bound at that size."""
    from row_reduction_amd.tune import COLD_BYTES, Case, GraphTimer, launches_per_graph
    out = []
    copy_cache = {}

    def copy_ceiling(rows, cols, cold, elem):
        """Per-call us of rr_copy_f32 reading and writing a rows x cols matrix
        of `elem`-byte elements (2 * elem * RC bytes), hot or cycling distinct
        buffers like the cold cases."""
        key = (rows, cols, cold, elem)
        if key not in copy_cache:
            n = max(1, rows * cols * elem // 4)
            nsets = max(2, min(1024, COLD_BYTES // (8 * n))) if cold else 1
            src = [torch.randn(n, device=device) for _ in range(nsets)]
            dst = [torch.empty(n, device=device) for _ in range(nsets)]
            it = [0]

            def call():
                i = it[0] = (it[0] + 1) % nsets
                rr.rr_copy_f32(src[i], dst[i])
            reps = max(nsets, 40 if n < (1 << 20) else 8)
            res = graph_us(torch, call, reps)
            copy_cache[key] = res["us"]
            del src, dst
        return copy_cache[key]
    pairs = [("rmsnorm", s) for s in [(1, 127), (17, 257), (64, 4096), (1024, 4096)]]
    pairs += [(op, s) for s in workloads.FAMILY_SHAPES for op in workloads.OPS if op != "rmsnorm"]
    pairs += [("rmsnorm_bf16", s) for s in [(1, 127), (17, 257), (64, 4096), (1024, 4096), (16384, 8192)]]
    pairs += [(op + "_bf16", s) for s in workloads.FAMILY_SHAPES for op in workloads.OPS if op != "rmsnorm"]
    for op, (rows, cols) in pairs:
        plan = rr.rr_select_plan(op, rows, cols)
        inherently_cold = False
        for hot in (True, False):
            if not hot and inherently_cold:
                break
            case = Case(torch, op, rows, cols, False, device, hot=hot)
            if not hot and not case.cold_possible:
                continue
            inherently_cold = hot and case.cold
            n = launches_per_graph(torch, case, plan)
            gt = GraphTimer(torch, case, plan, n)
            vals = sorted(gt.sample_us() for _ in range(samples))
            us = vals[len(vals) // 2]
            single = []
            if hot:
                for _ in range(21):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    case.launch(0, plan)
                    torch.cuda.synchronize()
                    single.append((time.perf_counter() - t0) * 1e6)
                single.sort()
            nbytes = workloads.algorithmic_bytes(op, rows, cols)
            gbps = nbytes / (us * 1e3)
            elem = 2 if op.endswith("_bf16") else 4
            cus = copy_ceiling(rows, cols, case.cold, elem)
            out.append({"op": op, "shape": f"{rows}x{cols}", "cache": "cold" if case.cold else "hot",
                        "us_per_op": round(us, 3), "min_us": round(vals[0], 3),
                        "max_us": round(vals[-1], 3), "launches_per_graph": n,
                        "rows_per_s": round(rows / (us * 1e-6), 1), "GBps": round(gbps, 1),
                        "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                        "single_call_us": round(single[len(single) // 2], 2) if single else None,
                        "copy_same_shape_us": round(cus, 3),
                        "copy_same_shape_GBps": round(2 * elem * rows * cols / (cus * 1e3), 1),
                        "plan": plan.as_dict()})
            del gt, case
            torch.cuda.empty_cache()
    return out


def device_info(torch) -> dict:
    """The GPU the numbers come from (name, ISA, compute units, memory)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "memory_GiB": round(p.total_memory / 2 ** 30, 1)}


def host_cores() -> int:
    """Host cores available to this process (capped at 16, a one-GPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def long_rows_table(torch, rr, device, samples: int = 11) -> list:
    """Few long rows: the plan the plain entry points use (one workgroup per
    row, register or streaming path) against the split-row plan the *_ws
    entry points select with a workspace, per call (graph-replayed), hot and
    cycling distinct buffers."""
    from row_reduction_amd import workloads
    from row_reduction_amd.tune import Case, GraphTimer, launches_per_graph
    out = []
    shapes = [(1, 1 << 20), (8, 1 << 18), (32, 65536)]
    for op in ("rmsnorm", "softmax", "row_sum", "rmsnorm_bf16"):
        opn = "sum" if op == "row_sum" else op
        for rows, cols in shapes:
            rec = {"op": opn, "shape": f"{rows}x{cols}"}
            for mode, ws in (("plain", False), ("split", True)):
                case = Case(torch, opn, rows, cols, False, device, hot=False, workspace=ws)
                plan = None
                n = launches_per_graph(torch, case, plan)
                gt = GraphTimer(torch, case, plan, n)
                vals = sorted(gt.sample_us() for _ in range(samples))
                us = vals[len(vals) // 2]
                nbytes = workloads.algorithmic_bytes(opn, rows, cols)
                chosen = rr.rr_select_plan(opn, rows, cols).as_dict() if not ws else None
                rec[mode] = {"us_per_op": round(us, 3), "GBps": round(nbytes / (us * 1e3), 1),
                             "cache": "cold" if case.cold else "hot",
                             "plan": chosen if chosen else "split (selected with workspace)"}
                del gt, case
                torch.cuda.empty_cache()
            rec["split_speedup"] = round(rec["plain"]["us_per_op"] / rec["split"]["us_per_op"], 3)
            out.append(rec)
    return out


def streaming_table(torch, rr, device, samples: int = 9) -> list:
    """Rows beyond the register path (vocabulary-size cross-entropy and
    softmax, 65536-column normalisations), many of them: the streaming plan
    the selector picks, per call (graph-replayed; every input here is larger
    than the last-level cache), next to a same-bytes copy."""
    from row_reduction_amd import workloads
    from row_reduction_amd.tune import Case, GraphTimer, launches_per_graph
    out = []
    cases = [("cross_entropy", 2048, 128256), ("cross_entropy_bf16", 2048, 128256),
             ("softmax", 2048, 128256), ("softmax_bf16", 2048, 128256),
             ("rmsnorm", 4096, 65536), ("layernorm", 4096, 65536)]
    for op, rows, cols in cases:
        case = Case(torch, op, rows, cols, False, device)
        plan = rr.rr_select_plan(op, rows, cols)
        n = launches_per_graph(torch, case, plan)
        gt = GraphTimer(torch, case, plan, n)
        vals = sorted(gt.sample_us() for _ in range(samples))
        us = vals[len(vals) // 2]
        del gt, case
        torch.cuda.empty_cache()
        nbytes = workloads.algorithmic_bytes(op, rows, cols)
        out.append({"op": op, "shape": f"{rows}x{cols}", "us_per_op": round(us, 3),
                    "GBps": round(nbytes / (us * 1e3), 1),
                    "frac_of_peak": round(nbytes / (us * 1e3) / PEAK_HBM_GBPS, 4),
                    "plan": plan.as_dict()})
    return out


def single_call_table(torch, rr, device, reps: int = 200) -> dict:
    """Latency of tiny calls. (1) One RMSNorm 1x127 call end to end: the C
    entry point called through ctypes with raw pointers, then the stream
    synchronised through the HIP runtime, so the figure is the library's
    launch plus the runtime's round trip (no torch wrapper); and the same
    through the Python binding. (2) The pages' operator-coverage set (five
    operators and RMSNorm on four small shapes, 24 calls) as 24 separate
    launches and as one rr_batch launch: per-set time from HIP-graph replay
    (GPU side) and end to end with one synchronisation."""
    import ctypes
    import statistics

    from row_reduction_amd import _capi, workloads
    L = _capi.lib()
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        hip = ctypes.CDLL(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "libamdhip64.so"))
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    x = torch.randn(1, 127, device=device)
    w = torch.rand(127, device=device) + 0.5
    y = torch.empty_like(x)
    xp, wp, yp = x.data_ptr(), w.data_ptr(), y.data_ptr()

    def e2e(fn, n):
        out = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            out.append((time.perf_counter() - t0) * 1e6)
        return statistics.median(out)

    def native():
        L.rmsnorm_f32(xp, wp, yp, 1, 127, 1e-6, stream)
        hip.hipStreamSynchronize(stream)

    def binding():
        rr.rmsnorm_f32(x, w, 1e-6, y=y)
        torch.cuda.synchronize()
    for _ in range(20):
        native()
        binding()
    res = {"rmsnorm_1x127_native_us": round(e2e(native, reps), 2),
           "rmsnorm_1x127_binding_us": round(e2e(binding, reps), 2)}

    def set_latency(shapes, prefix):
        """The six operators on each shape: separate launches against one batch."""
        probs, calls, ccalls = [], [], []
        keep = []
        for i, (rows, cols) in enumerate(shapes):
            d = workloads.family_inputs(rows, cols, 700 + i)
            t = {k: torch.from_numpy(v).to(device) for k, v in d.items()}
            keep.append(t)
            for op in workloads.OPS:
                kw = {}
                if op in ("rmsnorm", "layernorm", "residual_layernorm"):
                    kw.update(w=t["gamma"], eps=1e-6 if op == "rmsnorm" else 1e-5)
                if op in ("layernorm", "residual_layernorm"):
                    kw["beta"] = t["beta"]
                if op == "residual_layernorm":
                    kw["residual"] = t["residual"]
                if op == "cross_entropy":
                    kw["targets"] = t["targets"]
                p, outs = rr.batch_problem(op, t["x"], **kw)
                probs.append(p)
                keep.append(outs)

                xp_, op_ = t["x"].data_ptr(), op
                rows_, cols_ = t["x"].shape
                if op == "rmsnorm":
                    args = (xp_, t["gamma"].data_ptr(), outs["y"].data_ptr(), rows_, cols_, 1e-6)
                elif op == "sum":
                    args = (xp_, outs["out"].data_ptr(), rows_, cols_)
                elif op == "softmax":
                    args = (xp_, outs["y"].data_ptr(), rows_, cols_)
                elif op == "layernorm":
                    args = (xp_, t["gamma"].data_ptr(), t["beta"].data_ptr(), outs["y"].data_ptr(), rows_, cols_, 1e-5)
                elif op == "residual_layernorm":
                    args = (xp_, t["residual"].data_ptr(), t["gamma"].data_ptr(), t["beta"].data_ptr(),
                            outs["y"].data_ptr(), None, rows_, cols_, 1e-5)
                else:
                    args = (xp_, t["targets"].data_ptr(), outs["out"].data_ptr(), rows_, cols_)
                ccalls.append((getattr(L, {"sum": "row_sum"}.get(op_, op_) + "_f32"), args))

                def call(op=op, t=t, kw=kw, outs=outs):
                    if op == "rmsnorm":
                        rr.rmsnorm_f32(t["x"], kw["w"], kw["eps"], y=outs["y"])
                    elif op == "sum":
                        rr.row_sum_f32(t["x"], out=outs["out"])
                    elif op == "softmax":
                        rr.softmax_f32(t["x"], y=outs["y"])
                    elif op == "layernorm":
                        rr.layernorm_f32(t["x"], kw["w"], kw["beta"], kw["eps"], y=outs["y"])
                    elif op == "residual_layernorm":
                        rr.residual_layernorm_f32(t["x"], kw["residual"], kw["w"], kw["beta"], kw["eps"], y=outs["y"])
                    else:
                        rr.cross_entropy_f32(t["x"], kw["targets"], loss=outs["out"])
                calls.append(call)
        arr = (_capi.rr_problem * len(probs))(*probs)

        def separate():
            for c in calls:
                c()

        def batched():
            st = L.rr_batch(arr, len(probs), torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(f"rr_batch failed: {st}")

        def separate_c():
            for fn, args in ccalls:
                fn(*args, stream)
        sep = graph_us(torch, separate, 20)
        bat = graph_us(torch, batched, 20)

        def sync(fn):
            def f():
                fn()
                hip.hipStreamSynchronize(stream)
            return f
        for _ in range(10):
            sync(separate)()
            sync(separate_c)()
            sync(batched)()
        res.update({prefix + "_problems": len(probs),
                    prefix + "_separate_gpu_us": round(sep["us"], 2),
                    prefix + "_batched_gpu_us": round(bat["us"], 2),
                    prefix + "_separate_binding_e2e_us": round(e2e(sync(separate), 50), 2),
                    prefix + "_separate_c_e2e_us": round(e2e(sync(separate_c), 50), 2),
                    prefix + "_batched_c_e2e_us": round(e2e(sync(batched), reps), 2)})

    # The pages' operator-coverage set (24 problems), and its tiny part alone.
    set_latency(workloads.FAMILY_SHAPES, "coverage_set")
    set_latency(workloads.FAMILY_SHAPES[:2], "tiny_set")
    return res


def cpu_baseline(workloads, x_np, w_np, eps, y_gpu_sample, budget_s: float = 10.0) -> dict:
    """The CPU oracle, as it is (plain fp64 C loops), on row blocks of the
    headline input: first on one thread, then on every host core with a
    static row split (the oracle's C call releases the GIL), each leg for
    about half the time budget. Also checks the GPU output on the first block."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    rows, cols = x_np.shape
    block = 256
    first = oracle.rmsnorm(x_np[:block], w_np, eps)

    def leg(threads: int, seconds: float):
        t0 = time.perf_counter()
        done = 0
        r = 0
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            while time.perf_counter() - t0 < seconds:
                starts = [(r + i * block) % rows for i in range(threads)]
                list(ex.map(lambda s0: oracle.rmsnorm(x_np[s0:s0 + block], w_np, eps), starts))
                done += threads * block
                r = (r + threads * block) % rows
        return done, time.perf_counter() - t0

    cores = host_cores()
    d1, t1 = leg(1, budget_s * 0.4)
    dn, tn = leg(cores, budget_s * 0.6)
    gbps = lambda d, t: (8 * d * cols + 4 * cols) / t / 1e9
    err = np.abs(y_gpu_sample.astype(np.float64) - first.astype(np.float64))
    ok = bool(np.all(err <= 1e-5 + 1e-5 * np.abs(first.astype(np.float64))))
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(gbps(dn, tn), 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_op_full_shape": round(tn / dn * rows * 1e6, 1),
            "rows_per_s": round(dn / tn, 1),
            "single_thread_GBps": round(gbps(d1, t1), 3),
            "single_thread_rows_per_s": round(d1 / t1, 1),
            "sample": f"rmsnorm_f32 16384x8192 input in blocks of {block} rows: {dn} rows on "
                      f"{cores} threads in {tn:.1f} s, {d1} rows on 1 thread in {t1:.1f} s "
                      "(fp64 C loops, static row split)",
            "cpu_model": cpu, "gpu_matches_oracle_on_first_block": ok}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): rows are "
              "independent, so a multi-GPU run is row sharding with no communication and its "
              "per-GPU kernel is the one measured here at N=1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import row_reduction_amd as rr
    from row_reduction_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    rr._capi.lib()
    device = torch.device("cuda:0")
    rows, cols = HEADLINE

    log("generating 16384x8192 input")
    wl = [w for w in workloads.config_workloads(4) if (w.rows, w.cols) == HEADLINE][0]
    x = torch.from_numpy(wl.x).to(device)
    w = torch.from_numpy(wl.w).to(device)
    y = torch.empty_like(x)
    plan = rr.rr_select_plan("rmsnorm", rows, cols)
    nbytes = workloads.algorithmic_bytes("rmsnorm", rows, cols)

    def step():
        rr.rmsnorm_f32(x, w, wl.eps, y=y)

    log(f"warmup {args.warmup} steps, plan {plan.as_dict()}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timer = Timer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kernel_ms = timer.time_ms(step, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps: {wall * 1e3:.2f} ms wall, {kernel_ms:.2f} ms events")

    ms_per_step = wall * 1e3 / args.steps
    value = nbytes * args.steps / wall / 1e9
    avg_kernel_us = kernel_ms * 1e3 / args.steps
    achieved = nbytes / (avg_kernel_us * 1e3)
    src_hash = kernel_source_hash()
    traffic = counter_traffic(src_hash)

    # Same-bytes streaming copy (practical ceiling) and the empty-kernel floor.
    copy_src = x.view(-1)
    copy_dst = y.view(-1)
    copy = batch_us(torch, lambda: rr.rr_copy_f32(copy_src, copy_dst), rounds=1)
    empty = graph_us(torch, lambda: rr.rr_empty_kernel(), 200)
    copy_gbps = 8 * rows * cols / (copy["us"] * 1e3)

    y_sample = None
    if not args.no_cpu:
        step()
        torch.cuda.synchronize()
        y_sample = y[:256].cpu().numpy()
    shapes = [] if args.no_shapes else shape_table(torch, rr, workloads, device)
    long_rows = [] if args.no_shapes else long_rows_table(torch, rr, device)
    streaming = [] if args.no_shapes else streaming_table(torch, rr, device)
    single = {} if args.no_shapes else single_call_table(torch, rr, device)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_op": round(avg_kernel_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy: x~N(0,1), w~U(0.5,1.5))",
        "config": {"workload": "rmsnorm_f32 16384x8192, eps=1e-6", "rows": rows, "cols": cols,
                   "plan": plan.as_dict(), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "kernel_source_sha256": src_hash},
        "copy_ceiling": {"bytes": 8 * rows * cols, "us": round(copy["us"], 2),
                         "GBps": round(copy_gbps, 1), "frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4)},
        "launch_floor_us": round(empty["us"], 3),
        "device": device_info(torch),
        "shapes": shapes,
        "long_rows": long_rows,
        "streaming_rows": streaming,
        "single_call": single,
    }
    if not args.no_cpu:
        log(f"cpu baseline ({args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(workloads, wl.x, wl.w, wl.eps, y_sample, args.cpu_seconds)
        result["cpu_baseline"]["gpu_over_oracle"] = round(value / result["cpu_baseline"]["value"], 1)
    else:
        result["cpu_baseline"] = None
    _ = np
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

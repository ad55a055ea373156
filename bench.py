#!/usr/bin/env python3
"""Benchmark of the FP32 row-reduction library on one MI355X.

One step = one rmsnorm_f32 call (plan lookup, vectorised load, per-lane sum of
squares, wavefront and LDS reduction, rsqrt-scale epilogue and store) over the
bandwidth-bound 16384x8192 RMSNorm workload (x ~ N(0,1), w ~ U(0.5,1.5),
eps = 1e-6), inputs resident in HBM.

The LAST line on stdout is one compact JSON object (under 2 KB):

  value         whole-job throughput of the timed steps in algorithmic GB/s
                (bytes = 8*rows*cols + 4*cols per call: x read once, y
                written once, w read once)
  roofline      the RMSNorm kernel's achieved GB/s (algorithmic bytes /
                average kernel duration from HIP events on the launch stream)
                against MI355X's 8 TB/s HBM peak; `traffic` from hardware
                counters when a committed counter summary matches the current
                kernel source
  cpu_baseline  the CPU oracle timed on host cores over a bounded sample
  parity        how many timed configurations were checked in full against
                the oracle in this run, and how many failed

Everything else goes to a detail file (--detail, default
bench_detail.json in the working directory) and, one line per row, to stderr:

  shapes          per (operator, shape, cache state): GPU us/op (median of
                  graph-replayed samples, raw samples kept), rows/s, GB/s and
                  fraction of peak; the fastest same-bytes stream (copy, or
                  read-only for row sum and cross-entropy) over 12 geometries;
                  the CPU oracle's us/op on the same inputs (all cores used
                  and one core), the GPU/oracle speedup, and a full
                  element-by-element check of the GPU output against the
                  oracle taken before the row is timed
  long_rows       few long rows: one workgroup per row against split rows
  streaming_rows  many rows beyond the register path (vocabulary-size
                  cross-entropy and softmax, 65536-column normalisations)
  single_call     end-to-end latency of one tiny call, and the 24-call
                  operator-coverage set as separate launches against one
                  batched launch

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
# Host threads the CPU oracle may use: the host cores this process may run on,
# capped at 16, a one-GPU share of the GPU host's cores.
CPU_THREAD_CAP = 16
STREAM_GEOMETRIES = [(p, b) for p in (1, 2, 4, 8) for b in (256, 512, 1024)]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Fingerprint of the RMSNorm kernel as launched here: its device sources
    and the selected plan (the counter summary records the same)."""
    from row_reduction_amd.profile_cases import headline_fingerprint
    return headline_fingerprint()


def device_source_hash() -> str:
    """sha256 of every device source (what any row's timing depends on)."""
    from row_reduction_amd.tune import source_hash
    return source_hash()


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
    vals = [timer.time_ms(g.replay, 1) * 1000.0 / n for _ in range(samples)]
    s = sorted(vals)
    return {"us": s[len(s) // 2], "min_us": s[0], "max_us": s[-1], "samples_us": [round(v, 4) for v in vals]}


def device_info(torch) -> dict:
    """The GPU the numbers come from (name, ISA, compute units, memory)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "memory_GiB": round(p.total_memory / 2 ** 30, 1)}


def host_cores() -> tuple[int, int]:
    """(threads the oracle uses, host cores this process may run on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(CPU_THREAD_CAP, n)), n


def cpu_model() -> str:
    """The host CPU's model name, with its family, model and stepping numbers
    (which identify the generation where the name is generic, as it is on
    some virtual machines: family 25 is Zen 3/4, 26 is Zen 5)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        pass
    name = fields.get("model name") or platform.processor() or "unknown"
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


# ---- same-bytes stream ceiling ----------------------------------------------------

class Ceilings:
    """Fastest rr_stream_f32 geometry moving a given number of bytes: a copy
    (half read, half written) or a read-only stream, hot or cycling distinct
    buffers like the cold cases; per call, graph-replayed like the rows."""

    def __init__(self, torch, rr, device):
        self.torch, self.rr, self.device = torch, rr, device
        self.cache = {}

    def get(self, nbytes: int, read_only: bool, cold: bool) -> dict:
        from row_reduction_amd.tune import COLD_BYTES
        torch = self.torch
        n = max(4, nbytes // (4 if read_only else 8))
        # Sizes within about 1.6 % share one measurement (rows compare by GB/s).
        q = 1 << max(8, n.bit_length() - 7)
        n = -(-n // q) * q if n >= (1 << 16) else n
        key = (n, read_only, cold)
        if key in self.cache:
            return self.cache[key]
        per_set = 4 * n * (1 if read_only else 2)
        nsets = max(2, min(1024, -(-COLD_BYTES // per_set))) if cold else 1
        src = [torch.zeros(n, device=self.device) for _ in range(nsets)]
        # A read-only stream's sink needs one float per thread launched (at
        # most n / 4 + 1024); it is never written.
        dst = [torch.empty(n + (1024 if read_only else 0), device=self.device) for _ in range(nsets)]
        geoms = STREAM_GEOMETRIES if per_set >= (1 << 20) else [(1, 256), (8, 1024)]
        best = None
        for packs, block in geoms:
            it = [0]

            def call(packs=packs, block=block):
                i = it[0] = (it[0] + 1) % nsets
                self.rr.rr_stream_f32(src[i], dst[i], copy=not read_only, packs_per_thread=packs, block=block)
            reps = max(nsets, 40 if per_set < (1 << 22) else 8)
            res = graph_us(torch, call, reps, samples=7)
            if best is None or res["us"] < best["us"]:
                best = {"us": round(res["us"], 3), "packs_per_thread": packs, "block": block,
                        "kind": "read" if read_only else "copy", "bytes": per_set}
        best["GBps"] = round(best["bytes"] / (best["us"] * 1e3), 1)
        del src, dst
        torch.cuda.empty_cache()
        self.cache[key] = best
        return best


# ---- the CPU baseline leg: the only part of the benchmark that uses the oracle ----

class OracleLeg:
    """The CPU oracle as it is (plain fp64 C loops), run on the same seeded
    inputs as the GPU: over the whole matrix with a static row split on
    `cores` threads (its result is also the reference for a full check of the
    GPU output), and on one thread over a row sample scaled to the matrix."""

    def __init__(self, cores: int):
        import oracle
        self.oracle = oracle
        self.cores = cores

    def _fn(self, op: str, h: dict):
        o = self.oracle
        bf = op.endswith("_bf16")
        base = op[:-5] if bf else op
        sfx = "_bf16" if bf else ""
        if base == "rmsnorm":
            f = getattr(o, "rmsnorm" + sfx)
            return lambda a, b: {"y": f(h["x"][a:b], h["w"], h["eps"])}
        if base == "sum":
            f = getattr(o, "row_sum" + sfx)
            return lambda a, b: {"out": f(h["x"][a:b])}
        if base == "softmax":
            f = getattr(o, "softmax" + sfx)
            return lambda a, b: {"y": f(h["x"][a:b])}
        if base == "layernorm":
            f = getattr(o, "layernorm" + sfx)
            return lambda a, b: {"y": f(h["x"][a:b], h["w"], h["beta"], h["eps"])}
        if base == "residual_layernorm":
            f = getattr(o, "residual_layernorm" + sfx)
            return lambda a, b: {"y": f(h["x"][a:b], h["residual"][a:b], h["w"], h["beta"], h["eps"])[0]}
        f = getattr(o, "cross_entropy" + sfx)
        return lambda a, b: {"out": f(h["x"][a:b], h["targets"][a:b])}

    def reference(self, op: str, h: dict, rows: int):
        """Oracle outputs of the whole matrix and the seconds it took on
        min(cores, rows) threads (repeated to at least 50 ms, median)."""
        import concurrent.futures as cf

        import numpy as np
        fn = self._fn(op, h)
        threads = max(1, min(self.cores, rows))
        bounds = [rows * i // threads for i in range(threads + 1)]
        times, out = [], None
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            t_total = 0.0
            while not times or (t_total < 0.05 and len(times) < 50):
                t0 = time.perf_counter()
                parts = list(ex.map(lambda i: fn(bounds[i], bounds[i + 1]), range(threads)))
                dt = time.perf_counter() - t0
                times.append(dt)
                t_total += dt
                if out is None:
                    out = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
        times.sort()
        return out, times[len(times) // 2], threads

    def single_thread_s(self, op: str, h: dict, rows: int, cols: int) -> float:
        """Seconds for the whole matrix on one thread, from a row sample of
        about 2M elements, repeated to at least 30 ms."""
        fn = self._fn(op, h)
        k = max(1, min(rows, -(-(1 << 21) // cols)))
        times, total = [], 0.0
        while not times or (total < 0.03 and len(times) < 100):
            t0 = time.perf_counter()
            fn(0, k)
            dt = time.perf_counter() - t0
            times.append(dt)
            total += dt
        times.sort()
        return times[len(times) // 2] * rows / k

    def check(self, got: dict, ref: dict, bf16: bool) -> dict:
        """Every element: float outputs within 1e-5 + 1e-5 |ref|, bfloat16
        outputs within one bfloat16 ulp of the oracle + 1e-5; NaN where the
        oracle has NaN. Returns the element count and the worst err/bound."""
        import numpy as np
        o = self.oracle
        n, worst, bad = 0, 0.0, 0
        for k, r in ref.items():
            g = got[k]
            if g.shape != r.shape:
                return {"elements": 0, "ok": False, "error": f"{k}: shape {g.shape} vs {r.shape}"}
            gf, rf = g.reshape(-1), r.reshape(-1)
            step = 1 << 24
            for s in range(0, rf.size, step):
                if bf16 and k == "y":
                    gv = o.bf16_to_float(gf[s:s + step]).astype(np.float64)
                    rv = o.bf16_to_float(rf[s:s + step]).astype(np.float64)
                    e = np.floor(np.log2(np.maximum(np.abs(rv), 2.0 ** -133)))
                    bound = np.maximum(2.0 ** (e - 7), 2.0 ** -133) + 1e-5
                else:
                    gv = gf[s:s + step].astype(np.float64)
                    rv = rf[s:s + step].astype(np.float64)
                    bound = 1e-5 + 1e-5 * np.abs(rv)
                nan_r = np.isnan(rv)
                bad += int(np.count_nonzero(np.isnan(gv) != nan_r))
                ratio = np.where(nan_r, 0.0, np.abs(gv - rv) / bound)
                ratio = np.where(np.isnan(ratio), np.inf, ratio)
                bad += int(np.count_nonzero(ratio > 1.0))
                worst = max(worst, float(ratio.max(initial=0.0)))
                n += rf[s:s + step].size
        return {"elements": n, "max_err_over_bound": round(worst, 4), "ok": bad == 0}

    def timed_reference(self, op: str, h: dict, rows: int, cols: int, nbytes: int):
        """The oracle's outputs for the whole matrix, and its timings (all
        threads, and one thread) in the bench row's units."""
        ref, secs, threads = self.reference(op, h, rows)
        one = self.single_thread_s(op, h, rows, cols)
        # The baseline is the faster of the two (a thread pool costs more
        # than a tiny matrix takes on one thread).
        best_s, best_t = (secs, threads) if secs <= one else (one, 1)
        us = best_s * 1e6
        return ref, {"us_per_op": round(us, 2), "threads": best_t,
                     "us_per_op_all_threads": round(secs * 1e6, 2), "all_threads": threads,
                     "us_per_op_1thread": round(one * 1e6, 2),
                     "rows_per_s": round(rows / best_s, 1), "GBps": round(nbytes / (us * 1e3), 3)}

    def row(self, op: str, h: dict, rows: int, cols: int, got: dict, nbytes: int, gpu_us: float) -> dict:
        """Full check of `got` and the oracle's timings for one bench row."""
        ref, timing = self.timed_reference(op, h, rows, cols, nbytes)
        parity = self.check(got, ref, op.endswith("_bf16"))
        del ref
        return {"parity": parity,
                "oracle": dict(timing, gpu_speedup=round(timing["us_per_op"] / gpu_us, 1) if gpu_us else None)}

    def headline(self, x_np, w_np, eps, budget_s: float) -> dict:
        """The bounded CPU baseline of the headline: row blocks of the 16384 x
        8192 input, first on one thread, then on `cores` threads with a static
        row split (the oracle's C call releases the GIL), each leg for about
        half the time budget."""
        import concurrent.futures as cf
        rows, cols = x_np.shape
        block = 256

        def leg(threads: int, seconds: float):
            t0 = time.perf_counter()
            done = 0
            r = 0
            with cf.ThreadPoolExecutor(max_workers=threads) as ex:
                while time.perf_counter() - t0 < seconds:
                    starts = [(r + i * block) % rows for i in range(threads)]
                    list(ex.map(lambda s0: self.oracle.rmsnorm(x_np[s0:s0 + block], w_np, eps), starts))
                    done += threads * block
                    r = (r + threads * block) % rows
            return done, time.perf_counter() - t0

        d1, t1 = leg(1, budget_s * 0.4)
        dn, tn = leg(self.cores, budget_s * 0.6)
        gbps = lambda d, t: (8 * d * cols + 4 * cols) / t / 1e9
        return {"value": round(gbps(dn, tn), 3), "unit": "GB/s", "cores": self.cores, "kind": "oracle",
                "us_per_op": round(tn / dn * rows * 1e6, 1), "rows_per_s": round(dn / tn, 1),
                "single_thread_GBps": round(gbps(d1, t1), 3),
                "sample": f"rmsnorm 16384x8192 rows in 256-row blocks: {dn} rows on {self.cores} "
                          f"threads in {tn:.1f} s, {d1} on 1 in {t1:.1f} s"}


# ---- GPU tables ---------------------------------------------------------------

def gpu_output(torch, case) -> dict:
    """Set 0's output after the last launch, as numpy (bfloat16 as bits)."""
    import numpy as np
    out = case.output()
    base = case.base
    key = "out" if base in ("sum", "cross_entropy") else "y"
    if out.dtype == torch.bfloat16:
        return {key: out.view(torch.int16).cpu().numpy().view(np.uint16)}
    return {key: out.cpu().numpy()}


def time_case(torch, case, plan, samples: int) -> dict:
    from row_reduction_amd.tune import GraphTimer, launches_per_graph
    n = launches_per_graph(torch, case, plan)
    gt = GraphTimer(torch, case, plan, n)
    vals = [gt.sample_us() for _ in range(samples)]
    s = sorted(vals)
    del gt
    return {"us": s[len(s) // 2], "min_us": s[0], "max_us": s[-1], "launches_per_graph": n,
            "samples_us": [round(v, 4) for v in vals]}


def plan_str(plan) -> str:
    from row_reduction_amd.plans import plan_key
    return plan_key(plan)


def shape_table(torch, rr, workloads, device, ceilings, leg, src_hash, samples: int = 15) -> list:
    """Every measured (operator, shape) with the selected plan, hot and (for
    working sets of 1 MiB or more) cold, each row checked in full against the
    oracle before it is timed."""
    from row_reduction_amd.tune import Case
    out = []
    pairs = [("rmsnorm", s) for s in [(1, 127), (17, 257), (64, 4096), (1024, 4096)]]
    pairs += [(op, s) for s in workloads.FAMILY_SHAPES for op in workloads.OPS if op != "rmsnorm"]
    pairs += [("rmsnorm_bf16", s) for s in [(1, 127), (17, 257), (64, 4096), (1024, 4096), (16384, 8192)]]
    pairs += [(op + "_bf16", s) for s in workloads.FAMILY_SHAPES for op in workloads.OPS if op != "rmsnorm"]
    for op, (rows, cols) in pairs:
        plan = rr.rr_select_plan(op, rows, cols)
        nbytes = workloads.algorithmic_bytes(op, rows, cols)
        base = op[:-5] if op.endswith("_bf16") else op
        ref = timing = None
        inherently_cold = False
        for hot in (True, False):
            if not hot and inherently_cold:
                break
            case = Case(torch, op, rows, cols, False, device, hot=hot)
            if not hot and not case.cold_possible:
                continue
            inherently_cold = hot and case.cold
            # The output of this row's own buffers, checked before timing.
            case.launch(0, plan)
            torch.cuda.synchronize()
            parity = None
            if leg is not None:
                if ref is None:
                    ref, timing = leg.timed_reference(op, case.host, rows, cols, nbytes)
                parity = leg.check(gpu_output(torch, case), ref, op.endswith("_bf16"))
            t = time_case(torch, case, plan, samples)
            single = []
            if hot:
                for _ in range(21):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    case.launch(0, plan)
                    torch.cuda.synchronize()
                    single.append((time.perf_counter() - t0) * 1e6)
                single.sort()
            us = t["us"]
            gbps = nbytes / (us * 1e3)
            ceil = ceilings.get(nbytes, base in ("sum", "cross_entropy"), case.cold)
            row = {"op": op, "shape": f"{rows}x{cols}", "cache": "cold" if case.cold else "hot",
                   "us_per_op": round(us, 3), "min_us": round(t["min_us"], 3), "max_us": round(t["max_us"], 3),
                   "launches_per_graph": t["launches_per_graph"], "samples_us": t["samples_us"],
                   "rows_per_s": round(rows / (us * 1e-6), 1), "GBps": round(gbps, 1),
                   "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                   "single_call_us": round(single[len(single) // 2], 2) if single else None,
                   "stream_ceiling": ceil, "frac_of_ceiling": round(gbps / ceil["GBps"], 3),
                   "plan": plan_str(plan), "source_sha256": src_hash[:16]}
            if parity is not None:
                row["parity"] = parity
                row["oracle"] = dict(timing, gpu_speedup=round(timing["us_per_op"] / us, 1))
            out.append(row)
            log(row_line(row))
            del case
            torch.cuda.empty_cache()
    return out


def long_rows_table(torch, rr, device, leg, src_hash, samples: int = 11) -> list:
    """Few long rows: the plan the plain entry points use (one workgroup per
    row, register or streaming path) against the split-row plan the *_ws
    entry points select with a workspace, per call (graph-replayed), cycling
    distinct buffers; both outputs checked in full against the oracle."""
    from row_reduction_amd import workloads
    from row_reduction_amd.tune import Case
    out = []
    shapes = [(1, 1 << 20), (8, 1 << 18), (32, 65536)]
    for op in ("rmsnorm", "softmax", "row_sum", "rmsnorm_bf16"):
        opn = "sum" if op == "row_sum" else op
        for rows, cols in shapes:
            rec = {"op": opn, "shape": f"{rows}x{cols}", "source_sha256": src_hash[:16]}
            for mode, ws in (("plain", False), ("split", True)):
                case = Case(torch, opn, rows, cols, False, device, hot=False, workspace=ws)
                case.launch(0, None)
                torch.cuda.synchronize()
                got = gpu_output(torch, case) if leg is not None else None
                t = time_case(torch, case, None, samples)
                us = t["us"]
                nbytes = workloads.algorithmic_bytes(opn, rows, cols)
                rec[mode] = {"us_per_op": round(us, 3), "GBps": round(nbytes / (us * 1e3), 1),
                             "samples_us": t["samples_us"], "cache": "cold" if case.cold else "hot",
                             "plan": plan_str(rr.rr_select_plan(opn, rows, cols)) if not ws
                             else "split (selected with workspace)"}
                if got is not None:
                    chk = leg.row(opn, case.host, rows, cols, got, nbytes, us)
                    rec[mode]["parity"] = chk["parity"]
                    if mode == "plain":
                        rec["oracle"] = chk["oracle"]
                del case
                torch.cuda.empty_cache()
            rec["split_speedup"] = round(rec["plain"]["us_per_op"] / rec["split"]["us_per_op"], 3)
            out.append(rec)
            for mode in ("plain", "split"):
                p = rec[mode].get("parity")
                log(f"{rec['op']:>24} {rec['shape']:>12} {mode:>5}: {rec[mode]['us_per_op']:9.3f} us "
                    f"{rec[mode]['GBps']:8.1f} GB/s | parity {'-' if p is None else ('ok' if p['ok'] else 'FAILED')}")
    return out


def streaming_table(torch, rr, device, ceilings, leg, src_hash, samples: int = 9) -> list:
    """Rows beyond the register path (vocabulary-size cross-entropy and
    softmax, 65536-column normalisations), many of them: the streaming plan
    the selector picks, per call (graph-replayed; every input here is larger
    than the last-level cache), next to the same-bytes stream ceiling; each
    checked in full against the oracle."""
    from row_reduction_amd import workloads
    from row_reduction_amd.tune import Case
    out = []
    cases = [("cross_entropy", 2048, 128256), ("cross_entropy_bf16", 2048, 128256),
             ("softmax", 2048, 128256), ("softmax_bf16", 2048, 128256),
             ("rmsnorm", 4096, 65536), ("layernorm", 4096, 65536)]
    for op, rows, cols in cases:
        case = Case(torch, op, rows, cols, False, device)
        plan = rr.rr_select_plan(op, rows, cols)
        case.launch(0, plan)
        torch.cuda.synchronize()
        got = gpu_output(torch, case) if leg is not None else None
        t = time_case(torch, case, plan, samples)
        us = t["us"]
        nbytes = workloads.algorithmic_bytes(op, rows, cols)
        base = op[:-5] if op.endswith("_bf16") else op
        row = {"op": op, "shape": f"{rows}x{cols}", "us_per_op": round(us, 3), "samples_us": t["samples_us"],
               "GBps": round(nbytes / (us * 1e3), 1), "frac_of_peak": round(nbytes / (us * 1e3) / PEAK_HBM_GBPS, 4),
               "plan": plan_str(plan), "source_sha256": src_hash[:16]}
        host = case.host
        del case
        torch.cuda.empty_cache()
        ceil = ceilings.get(nbytes, base in ("sum", "cross_entropy"), True)
        row["stream_ceiling"] = ceil
        row["frac_of_ceiling"] = round(row["GBps"] / ceil["GBps"], 3)
        if got is not None:
            row.update(leg.row(op, host, rows, cols, got, nbytes, us))
        out.append(row)
        log(row_line(row))
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


def row_line(r: dict) -> str:
    """One stderr line per bench row."""
    par = r.get("parity")
    p = "parity -" if par is None else (f"parity ok ({par['elements']} el, max {par['max_err_over_bound']})"
                                        if par["ok"] else "PARITY FAILED")
    o = r.get("oracle")
    oc = "" if o is None else f" | oracle {o['us_per_op']} us ({o['threads']} thr), x{o['gpu_speedup']}"
    c = r.get("stream_ceiling")
    cc = "" if c is None else f" | ceiling {c['us']} us ({r['frac_of_ceiling']:.2f})"
    return (f"{r['op']:>24} {r['shape']:>12} {r.get('cache', 'cold'):>4}: {r['us_per_op']:9.3f} us "
            f"{r['GBps']:8.1f} GB/s{cc}{oc} | {p} | {r['plan']}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape, long-row, streaming "
                                                             "and single-call tables")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (baseline and parity checks)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--detail", default="bench_detail.json",
                    help="where the full result (every table) is written")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): rows are "
              "independent, so a multi-GPU run is row sharding with no communication and its "
              "per-GPU kernel is the one measured here at N=1.", file=sys.stderr)
        return 2

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

    log(f"warmup {args.warmup} steps, plan {plan_str(plan)}")
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
    kernel_hash = kernel_source_hash()
    src_hash = device_source_hash()
    traffic = counter_traffic(kernel_hash)

    # rr_copy_f32 over the same 2^30 bytes: the calibration kernel of the
    # hardware byte counters (its reads and writes are known exactly).
    calib = graph_us(torch, lambda: rr.rr_copy_f32(x.view(-1), y.view(-1)), 8, samples=5)
    ceilings = Ceilings(torch, rr, device)
    head_ceiling = ceilings.get(nbytes, False, True)
    empty = graph_us(torch, lambda: rr.rr_empty_kernel(), 200)
    log(f"headline {avg_kernel_us:.2f} us/launch = {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBPS:.3f} of peak); "
        f"fastest same-bytes copy {head_ceiling['us']} us ({head_ceiling['packs_per_thread']} packs x "
        f"{head_ceiling['block']}); launch floor {empty['us']:.3f} us")

    cores, cores_avail = host_cores()
    leg = None if args.no_cpu else OracleLeg(cores)
    head_parity = None
    if leg is not None:
        log("headline: full oracle check of the output")
        step()  # y again (the calibration copy above overwrote it)
        torch.cuda.synchronize()
        y_np = y.cpu().numpy()
        ref, secs, threads = leg.reference("rmsnorm", {"x": wl.x, "w": wl.w, "eps": wl.eps}, rows)
        head_parity = leg.check({"y": y_np}, ref, False)
        del ref, y_np
        log(f"headline parity: {head_parity}")

    shapes = long_rows = streaming = []
    single = {}
    if not args.no_shapes:
        shapes = shape_table(torch, rr, workloads, device, ceilings, leg, src_hash)
        long_rows = long_rows_table(torch, rr, device, leg, src_hash)
        streaming = streaming_table(torch, rr, device, ceilings, leg, src_hash)
        single = single_call_table(torch, rr, device)
        log(f"single call: {single}")

    cpu = None
    if leg is not None:
        log(f"cpu baseline ({args.cpu_seconds:.0f} s)")
        cpu = leg.headline(wl.x, wl.w, wl.eps, args.cpu_seconds)
        cpu["cores_available"] = cores_avail
        cpu["cpu_model"] = cpu_model()
        cpu["gpu_over_oracle"] = round(value / cpu["value"], 1)

    checks = [r.get("parity") for r in shapes + streaming]
    checks += [r[m].get("parity") for r in long_rows for m in ("plain", "split")]
    checks = [c for c in checks if c is not None] + ([head_parity] if head_parity else [])
    failed = sum(1 for c in checks if not c["ok"])

    detail = {
        "metric": METRIC, "source_sha256": src_hash, "kernel_fingerprint": kernel_hash,
        "headline": {"us_per_launch": avg_kernel_us, "GBps": achieved, "parity": head_parity,
                     "plan": plan_str(plan)},
        "stream_ceiling": head_ceiling, "launch_floor_us": round(empty["us"], 3),
        "copy_2p30_bytes_us": round(calib["us"], 3),
        "device": device_info(torch), "cpu_baseline": cpu,
        "shapes": shapes, "long_rows": long_rows, "streaming_rows": streaming, "single_call": single,
    }
    if args.detail:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as f:
            json.dump(detail, f)
        log(f"detail written to {args.detail}")

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
                   "plan": plan_str(plan), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "kernel_source_sha256": kernel_hash[:16]},
        "stream_ceiling_us": head_ceiling["us"],
        "cpu_baseline": None if cpu is None else {
            k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample", "us_per_op", "rows_per_s",
                                "cores_available", "cpu_model")},
        "parity": {"checked": len(checks), "failed": failed,
                   "headline_max_err_over_bound": head_parity["max_err_over_bound"] if head_parity else None},
        "detail": args.detail,
    }
    line = json.dumps(result, ensure_ascii=False)
    if len(line.encode()) > 2048:
        raise SystemExit(f"headline JSON line is {len(line.encode())} bytes; keep it under 2 KB")
    print(line, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Kernel-duration profile of every measured (operator, shape) under rocprofv3.

`run` launches each case with the plan the library selects — warm-up launches
first, then `--launches` measured ones from one HIP graph, cache-hot (one buffer set) and, for
working sets of 1 MiB or more, cache-cold (cycling >= 768 MiB of distinct
buffers) — plus the library's same-bytes streaming copy and empty kernel, and
writes a manifest of what it launched, in order. Run it under

  rocprofv3 --kernel-trace --output-format csv -d OUT -o cases -- \\
      python3 <repo>/row_reduction_amd/profile_cases.py run --manifest OUT/manifest.json

Options: `--isolated` issues each measured launch as its own synchronised
call (the kernel starts on an idle GPU; nothing overlaps its start or its
drain); `--all-plans` runs every legal plan of each case, not only the
selected one; `--ceilings` adds rr_stream_f32 in every geometry moving each
case's algorithmic bytes (a copy, or a read-only stream for row sum and
cross-entropy), rotated over buffers the same way.

`summarize` then walks the trace's dispatches of librowred kernels in
dispatch order, attributes them to the manifest's cases (checking each
dispatch's grid size against the case's), and prints a markdown table of
kernel durations with algorithmic GB/s and the fraction of the 8 TB/s HBM
peak, and for graph runs the span per launch (first start to last end over
the launch count; under the profiler a graph's launches run spaced apart,
so short kernels start on an idle GPU):

  python3 <repo>/row_reduction_amd/profile_cases.py summarize OUT/manifest.json OUT/cases_kernel_trace.csv

Counter summaries, from `rocprofv3 --pmc` runs (one counter block per run):
`counters` gives the headline kernel's HBM traffic from FETCH_SIZE and
WRITE_SIZE runs of bench.py, calibrated by rr_copy_f32 of known bytes;
`counters-cases` the same per case of a `run --ceilings` manifest,
calibrated by that run's largest stream copy; `counters-table` lays out any
counters of such a run per case, with GRBM_GUI_ACTIVE net of the empty
kernel's, per XCD, and derived waves per CU and texture-address busy
fraction.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0

# The device sources the headline RMSNorm kernel instance is compiled from.
KERNEL_SOURCES = ("device.h", "internal.h", "kernels_rmsnorm.hip")


def kernel_fingerprint(plan: dict) -> str:
    """sha256 of the headline RMSNorm kernel as launched: its device sources
    and the plan it is launched with (which fixes the instance, the grid and
    the block). Counter readings stay valid while this is unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(KERNEL_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    h.update(json.dumps(plan, sort_keys=True).encode())
    return h.hexdigest()


def headline_fingerprint() -> str:
    """kernel_fingerprint of RMSNorm 16384x8192 with the plan the library selects."""
    import row_reduction_amd as rr
    return kernel_fingerprint(rr.rr_select_plan("rmsnorm", 16384, 8192).as_dict())


def cases_list(shapes_only=None, ops_only=None):
    from row_reduction_amd import workloads
    cases = [("rmsnorm", s) for s in [(1, 127), (17, 257), (64, 4096), (1024, 4096), (16384, 8192)]]
    cases += [(op, s) for s in workloads.FAMILY_SHAPES for op in workloads.OPS if op != "rmsnorm"]
    cases += [("rmsnorm_bf16", s) for s in [(1024, 4096), (16384, 8192)]]
    cases += [(op + "_bf16", (1024, 4096)) for op in workloads.OPS if op != "rmsnorm"]
    # Streaming path: vocabulary-size rows and 65536-column normalisations.
    cases += [("cross_entropy", (2048, 128256)), ("cross_entropy_bf16", (2048, 128256)),
              ("softmax", (2048, 128256)), ("softmax_bf16", (2048, 128256)),
              ("rmsnorm", (4096, 65536)), ("layernorm", (4096, 65536)),
              ("residual_layernorm", (4096, 65536)), ("rmsnorm_bf16", (4096, 65536)),
              ("layernorm_bf16", (4096, 65536)), ("residual_layernorm_bf16", (4096, 65536))]
    if shapes_only:
        cases = [c for c in cases if f"{c[1][0]}x{c[1][1]}" in shapes_only]
    if ops_only:
        cases = [c for c in cases if c[0] in ops_only]
    return cases


def run(args) -> int:
    import torch

    import row_reduction_amd as rr
    from row_reduction_amd import plans as plans_mod
    from row_reduction_amd import workloads
    from row_reduction_amd.tune import COLD_BYTES, Case

    rr._capi.lib()
    device = torch.device("cuda:0")
    manifest = {"launches": args.launches, "warmup": args.warmup, "isolated": bool(args.isolated),
                "entries": []}

    def add(name, kind, count, grid, nbytes, warm, extra=None):
        e = {"name": name, "kind": kind, "count": count, "grid_size": grid, "bytes": nbytes,
             "warmup": warm}
        if extra:
            e.update(extra)
        manifest["entries"].append(e)

    def measured(launch, first):
        """The measured launches: back to back from one HIP graph, or (isolated)
        one launch per synchronised call, so each kernel starts on an idle GPU
        and nothing overlaps its start or its drain."""
        if args.isolated:
            for i in range(args.launches):
                launch(first + i)
                torch.cuda.synchronize()
            return
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.launches):
                launch(first + i)
        graph.replay()
        torch.cuda.synchronize()
        del graph

    ceilings_done = set()

    def ceilings(nbytes, read_only, cold):
        """rr_stream_f32 of every geometry moving `nbytes` (a copy: half read,
        half written; read-only: all read), rotated over distinct buffers like
        the cold cases."""
        n = max(4, nbytes // (4 if read_only else 8))
        key = (n, read_only, cold)
        if key in ceilings_done:
            return
        ceilings_done.add(key)
        per_set = 4 * n * (1 if read_only else 2)
        nsets = max(1, min(1024, -(-COLD_BYTES // per_set))) if cold else 1
        src = [torch.zeros(n, device=device) for _ in range(nsets)]
        dst = [torch.empty(n + (1024 if read_only else 0), device=device) for _ in range(nsets)]
        for packs in (1, 2, 4, 8):
            for block in (256, 512, 1024):
                groups = max(1, -(-(n // 4) // (packs * block)))
                label = (f"stream {'read' if read_only else 'copy'} {4 * n * (1 if read_only else 2)} B "
                         f"{'cold' if cold else 'hot'} packs{packs} b{block}")

                def launch(i, packs=packs, block=block):
                    k = i % nsets
                    rr.rr_stream_f32(src[k], dst[k], copy=not read_only, packs_per_thread=packs, block=block)
                warm = max(args.warmup, nsets)
                for i in range(warm):
                    launch(i)
                add(label, "stream", warm, groups * block, 4 * n * (1 if read_only else 2), True)
                torch.cuda.synchronize()
                measured(launch, warm)
                add(label, "stream", args.launches, groups * block, 4 * n * (1 if read_only else 2), False)
        del src, dst
        torch.cuda.empty_cache()

    for op, (rows, cols) in cases_list(args.shapes, args.ops):
        selected = rr.rr_select_plan(op, rows, cols)
        plan_list = [selected]
        if args.all_plans:
            plan_list = plans_mod.candidate_plans(op, rows, cols, caches=(0, 1, 2))
        nbytes = workloads.algorithmic_bytes(op, rows, cols)
        inherently_cold = False
        for hot in (True, False):
            if not hot and inherently_cold:
                break
            case = Case(torch, op, rows, cols, False, device, hot=hot)
            if not hot and not case.cold_possible:
                continue
            inherently_cold = hot and case.cold
            if hot and args.cold_only and case.cold_possible and not case.cold:
                del case
                continue
            for plan in plan_list:
                groups = -(-rows // plan.rows_per_group)
                grid = groups * plan.block
                tag = "" if not args.all_plans else " " + plans_mod.plan_key(plan) + \
                    (" (selected)" if plan.as_dict() == selected.as_dict() else "")
                label = f"{op} {rows}x{cols} {'cold' if case.cold else 'hot'}{tag}"
                print(f"case {label} plan {plan.as_dict()}", flush=True)
                n_warm = max(args.warmup, case.nsets)
                for i in range(n_warm):
                    case.launch(i, plan)
                add(label, "op", n_warm, grid, nbytes, True)
                torch.cuda.synchronize()
                measured(lambda i, plan=plan: case.launch(i, plan), n_warm)
                add(label, "op", args.launches, grid, nbytes, False, {"plan": plan.as_dict()})
            if args.ceilings:
                base = op[:-5] if op.endswith("_bf16") else op
                ceilings(nbytes, base in ("sum", "cross_entropy"), case.cold)
            del case
            torch.cuda.empty_cache()

    if not args.no_reference:
        # Same-bytes streaming copy (1 GiB moved) and the empty kernel.
        n = 16384 * 8192
        src = torch.zeros(n, dtype=torch.float32, device=device)
        dst = torch.empty_like(src)
        copy_grid = -(-(n // 4) // 256) * 256   # one float4 per thread, 256-thread groups
        for name, kind, fn, grid, nbytes in (
                ("rr_copy_f32 2^27 floats", "copy", lambda i: rr.rr_copy_f32(src, dst), copy_grid, 8 * n),
                ("rr_empty_kernel", "empty", lambda i: rr.rr_empty_kernel(), 64, 0)):
            for i in range(args.warmup):
                fn(i)
            add(name, kind, args.warmup, grid, nbytes, True)
            torch.cuda.synchronize()
            measured(fn, 0)
            add(name, kind, args.launches, grid, nbytes, False)
    os.makedirs(os.path.dirname(os.path.abspath(args.manifest)), exist_ok=True)
    with open(args.manifest, "w") as f:
        json.dump(manifest, f)
    print(f"wrote {args.manifest}", flush=True)
    return 0


def ours(name: str) -> bool:
    # The profiler leaves some names mangled (e.g. instances over __bf16).
    return ("rowred::" in name or name.startswith("_ZN6rowred") or "copy_kernel" in name
            or "empty_kernel" in name or "stream_kernel" in name)


def demangle(name: str) -> str:
    """Readable name of a librowred kernel instance (template arguments in
    order; bfloat16 shown as bf16), whether or not the trace demangled it."""
    import re
    if not name.startswith("_Z"):
        # The profiler's own demangling reads a bfloat16 argument followed by
        # `true` (DF16bLb1E) as these three.
        return name.replace("bool _Accum, bool, E>", "bf16, true>")
    m = re.match(r"_ZN6rowred(\d+)(\w+?)I(.*)EEvNS_4ArgsE$", name)
    if not m:
        return name
    kernel = m.group(2)[: int(m.group(1))]
    args = []
    for tok in re.findall(r"Li(-?\d+)E|Lb([01])E|(DF16b)|(f)(?=E|$)", m.group(3)):
        if tok[0]:
            args.append(tok[0])
        elif tok[1]:
            args.append("true" if tok[1] == "1" else "false")
        elif tok[2]:
            args.append("bf16")
        else:
            args.append("float")
    return f"{kernel}<{', '.join(args)}>(Args)"


def summarize(args) -> int:
    man = json.load(open(args.manifest))
    rows = [r for r in csv.DictReader(open(args.trace)) if ours(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    pos = 0
    out = []
    for e in man["entries"]:
        chunk = rows[pos:pos + e["count"]]
        pos += e["count"]
        if len(chunk) != e["count"]:
            raise SystemExit(f"trace ended early at {e['name']}")
        for r in chunk:
            if int(r.get("Grid_Size") or r["Grid_Size_X"]) != e["grid_size"]:
                raise SystemExit(f"dispatch {r['Dispatch_Id']} grid {r.get('Grid_Size') or r['Grid_Size_X']} does not match "
                                 f"{e['name']} ({e['grid_size']})")
        if e["warmup"]:
            continue
        durs = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in chunk)
        med = statistics.median(durs)
        avg = sum(durs) / len(durs)
        gbps = e["bytes"] / med if e["bytes"] else None
        # The span from the first start to the last end over the launch
        # count: how far apart the profiled launches ran (under the profiler
        # a graph's launches are spaced by its per-dispatch work).
        span = (max(int(r["End_Timestamp"]) for r in chunk) - min(int(r["Start_Timestamp"]) for r in chunk)) / len(chunk)
        out.append((e, chunk[0]["Kernel_Name"], len(durs), avg, med, durs[0], durs[-1], gbps, span))
    if pos != len(rows):
        raise SystemExit(f"{len(rows) - pos} librowred dispatches left unattributed")
    spans = not man.get("isolated", False)
    head = "| Case | Kernel | Launches | Avg ns | Median ns | Min ns | Max ns | GB/s (median) | % of 8 TB/s |"
    rule = "|---|---|---:|---:|---:|---:|---:|---:|---:|"
    if spans:
        head += " Span per launch ns |"
        rule += "---:|"
    print(head)
    print(rule)
    for e, kname, n, avg, med, lo, hi, gbps, span in out:
        k = demangle(kname).replace("rowred::", "").replace("(rowred::Args)", "").replace("void ", "")
        k = k.replace("(anonymous namespace)::", "")
        g = f"{gbps:.1f}" if gbps else "—"
        f = f"{100 * gbps / PEAK_GBPS:.1f}" if gbps else "—"
        line = f"| {e['name']} | `{k}` | {n} | {avg:.0f} | {med:.0f} | {lo} | {hi} | {g} | {f} |"
        if spans:
            line += f" {span:.0f} |"
        print(line)
    return 0


def counters(args) -> int:
    """Calibrated HBM traffic per launch of the headline RMSNorm kernel from two
    rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --no-shapes --no-cpu`, which also launches rr_copy_f32 over the
    same 2^27 floats: each counter is scaled by (bytes the copy must move) /
    (what the counter reads for the copy)."""

    def load(path, counter):
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return per

    fetch = load(args.fetch_csv, "FETCH_SIZE")
    write = load(args.write_csv, "WRITE_SIZE")
    n = 16384 * 8192
    copy_name = [k for k in fetch if "copy_kernel" in k][0]
    rms_name = [k for k in fetch if k.startswith("void rowred::reg_kernel<0,")][0]
    avg = lambda v: sum(v) / len(v)
    f_copy, w_copy = avg(fetch[copy_name]) * 1024, avg(write[copy_name]) * 1024
    f_scale, w_scale = 4 * n / f_copy, 4 * n / w_copy
    f_rms, w_rms = avg(fetch[rms_name]) * 1024 * f_scale, avg(write[rms_name]) * 1024 * w_scale
    algorithmic = 8 * n + 4 * 8192
    print(f"Kernel: `{rms_name}` (rmsnorm_f32 16384x8192, plan from the measured table)")
    print()
    print("| Counter | Copy kernel raw (KiB/dispatch) | Copy bytes known | Scale | RMSNorm raw (KiB/dispatch) | RMSNorm calibrated bytes |")
    print("|---|---:|---:|---:|---:|---:|")
    print(f"| FETCH_SIZE | {f_copy / 1024:.1f} | {4 * n} | {f_scale:.4f} | {avg(fetch[rms_name]):.1f} | {f_rms:.0f} |")
    print(f"| WRITE_SIZE | {w_copy / 1024:.1f} | {4 * n} | {w_scale:.4f} | {avg(write[rms_name]):.1f} | {w_rms:.0f} |")
    print()
    print(f"Algorithmic bytes per launch: {algorithmic}; calibrated traffic / algorithmic = "
          f"{(f_rms + w_rms) / algorithmic:.4f}.")
    print()
    print(f"source_sha256: {headline_fingerprint()}")
    print(f"traffic_bytes_per_launch: {f_rms + w_rms:.0f}")
    return 0


def counters_cases(args) -> int:
    """Per-case HBM traffic from two rocprofv3 --pmc runs of the same `run`
    command (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), dispatches
    attributed to the manifest's cases in order as in `summarize`. Each
    counter is scaled by what it reads for the manifest's largest stream copy
    (rr_stream_f32, --ceilings), whose reads and writes are each half of its
    known bytes."""
    man = json.load(open(args.manifest))

    def per_entry(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if ours(r["Kernel_Name"]) and r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        out, pos = [], 0
        for e in man["entries"]:
            chunk = rows[pos:pos + e["count"]]
            pos += e["count"]
            if len(chunk) != e["count"]:
                raise SystemExit(f"{counter}: trace ended early at {e['name']}")
            out.append(sum(float(r["Counter_Value"]) for r in chunk) * 1024 / len(chunk))
        if pos != len(rows):
            raise SystemExit(f"{counter}: {len(rows) - pos} dispatches left unattributed")
        return out

    fetch = per_entry(args.fetch_csv, "FETCH_SIZE")
    write = per_entry(args.write_csv, "WRITE_SIZE")
    copies = [(i, e) for i, e in enumerate(man["entries"]) if e["kind"] == "stream" and "copy" in e["name"]
              and not e["warmup"]]
    if not copies:
        raise SystemExit("the manifest holds no stream copy (run with --ceilings)")
    ci, ce = max(copies, key=lambda ie: ie[1]["bytes"])
    f_scale, w_scale = (ce["bytes"] / 2) / fetch[ci], (ce["bytes"] / 2) / write[ci]
    print(f"Calibration: `{ce['name']}` must read and write {ce['bytes'] // 2} B each; "
          f"FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}.")
    print()
    print("| Case | Algorithmic B | FETCH_SIZE calibrated B | WRITE_SIZE calibrated B | traffic / algorithmic |")
    print("|---|---:|---:|---:|---:|")
    for i, e in enumerate(man["entries"]):
        if e["warmup"] or not e["bytes"]:
            continue
        f, w = fetch[i] * f_scale, write[i] * w_scale
        print(f"| {e['name']} | {e['bytes']} | {f:.0f} | {w:.0f} | {(f + w) / e['bytes']:.4f} |")
    return 0


def counters_table(args) -> int:
    """Mean of every counter of one rocprofv3 --pmc run per manifest case
    (dispatches attributed in order as in `summarize`), with what they give
    per kernel. GRBM_GUI_ACTIVE is summed over the XCDs and, under counter
    collection, carries a fixed overhead that the manifest's empty kernel
    shows; the kernel's own active cycles per XCD are (GRBM_GUI_ACTIVE -
    empty kernel's) / XCDs. From them: waves resident per CU on average
    (SQ_WAVE_CYCLES / (active cycles x CUs)) and the fraction of the active
    cycles the busiest texture-address unit (which every vector memory
    access passes) was busy (TA_BUSY_max / active cycles)."""
    man = json.load(open(args.manifest))
    rows = [r for r in csv.DictReader(open(args.csv)) if ours(r["Kernel_Name"])]
    names = sorted({r["Counter_Name"] for r in rows})
    by_dispatch = {}
    for r in rows:
        by_dispatch.setdefault(int(r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(by_dispatch)
    pos = 0
    means = []
    for e in man["entries"]:
        chunk = ids[pos:pos + e["count"]]
        pos += e["count"]
        if len(chunk) != e["count"]:
            raise SystemExit(f"counters ended early at {e['name']}")
        if not e["warmup"]:
            means.append((e, {n: sum(by_dispatch[i].get(n, 0.0) for i in chunk) / len(chunk) for n in names}))
    if pos != len(ids):
        raise SystemExit(f"{len(ids) - pos} dispatches left unattributed")
    base = next((m.get("GRBM_GUI_ACTIVE", 0.0) for e, m in means if e["kind"] == "empty"), 0.0)
    print(f"Empty kernel's GRBM_GUI_ACTIVE (collection overhead, subtracted): {base:.0f}; XCDs {args.xcd}, CUs {args.cus}.")
    print()
    print("| Case | " + " | ".join(names) + " | active cycles per XCD | waves per CU | TA busy / active |")
    print("|---|" + "---:|" * (len(names) + 3))
    for e, m in means:
        act = (m.get("GRBM_GUI_ACTIVE", 0.0) - base) / args.xcd
        occ = m.get("SQ_WAVE_CYCLES", 0.0) / (act * args.cus) if act > 0 else float("nan")
        ta = m.get("TA_BUSY_max", 0.0) / act if act > 0 else float("nan")
        print(f"| {e['name']} | " + " | ".join(f"{m[n]:.0f}" for n in names) +
              f" | {act:.0f} | {occ:.2f} | {ta:.3f} |")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--manifest", required=True)
    r.add_argument("--launches", type=int, default=50)
    r.add_argument("--warmup", type=int, default=5)
    r.add_argument("--shapes", default=None, help="comma-separated subset, e.g. 1024x4096")
    r.add_argument("--ops", default=None, help="comma-separated subset, e.g. rmsnorm,cross_entropy_bf16")
    r.add_argument("--isolated", action="store_true",
                   help="one measured launch per synchronised call instead of a graph of back-to-back launches")
    r.add_argument("--all-plans", action="store_true", help="every legal plan (all cache policies), not only the selected one")
    r.add_argument("--ceilings", action="store_true",
                   help="also every rr_stream_f32 geometry moving each case's bytes")
    r.add_argument("--cold-only", action="store_true", help="skip the cache-hot runs of cases that can be cold")
    r.add_argument("--no-reference", action="store_true", help="skip the 1 GiB copy and the empty kernel")
    s = sub.add_parser("summarize")
    s.add_argument("manifest")
    s.add_argument("trace")
    c = sub.add_parser("counters")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    cc = sub.add_parser("counters-cases")
    cc.add_argument("manifest")
    cc.add_argument("fetch_csv")
    cc.add_argument("write_csv")
    ct = sub.add_parser("counters-table")
    ct.add_argument("manifest")
    ct.add_argument("csv")
    ct.add_argument("--cus", type=int, default=256)
    ct.add_argument("--xcd", type=int, default=8)
    args = ap.parse_args()
    if args.cmd == "counters-table":
        return counters_table(args)
    if args.cmd == "counters":
        return counters(args)
    if args.cmd == "counters-cases":
        return counters_cases(args)
    if args.cmd == "run":
        if args.shapes:
            args.shapes = set(args.shapes.split(","))
        if args.ops:
            args.ops = set(args.ops.split(","))
        return run(args)
    return summarize(args)


if __name__ == "__main__":
    sys.exit(main())

"""Split-row selector of the *_ws entry points: whether to cut a few long rows
into slices spread over many workgroups, and how wide a slice is.

The LuisaCompute notes ("Consecutive-worker reduction layout checkpoint",
section "Evidence and what remains") leave the spreading of one long row over
several workers as the next step; whether it pays depends on the shape. With
fewer than 256 rows the plain plans run one workgroup per row, so their time
grows with the row length and hardly with the row count, while a split plan
keeps the whole chip busy but pays a second launch and re-reads its slice:

  plain:  t_p = a + b * cols + e * rows * cols
  split:  t_s = c + d * rows * cols

per operator, in microseconds per call. The five constants of each operator
are fitted (least squares on relative error) to GPU timings of both kinds of
plan over a grid of (rows, cols), and frozen into csrc/split_model.inc; the
C++ selector evaluates the same two lines and splits iff t_s < t_p.

The slice width is a rule, applied before the comparison (the split timings
fitted are those of the slice the rule picks): the narrowest workgroup (64 to
1024 lanes, 16 slots per lane) that cuts a row into at most SLICE_MAX slices
with at most GROUPS_MAX workgroups in all, else 1024 lanes x 32 slots.

  python -m row_reduction_amd.split_model --measure OUT.json --ops rmsnorm,... \
      [--cols 8192,...] [--rows 1,2,...]                       # GPU: time a grid
  python -m row_reduction_amd.split_model --export OUT.csv grid.json [...]
  python -m row_reduction_amd.split_model --fit row_reduction_amd/data/split_timings.csv --emit
  python -m row_reduction_amd.split_model --report row_reduction_amd/data/split_timings.csv \\
      row_reduction_amd/data/split_heldout.csv
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DATA = os.path.join(HERE, "data", "split_timings.csv")
HELDOUT = os.path.join(HERE, "data", "split_heldout.csv")
INC = os.path.join(HERE, "csrc", "split_model.inc")

# Operators in rr_op order (the rows of split_model.inc).
OPS = ["rmsnorm", "sum", "softmax", "layernorm", "residual_layernorm", "cross_entropy"]
OPS = OPS + [o + "_bf16" for o in OPS]
ROWS_LIMIT = 256       # split only below this many rows (plain plans fill the chip from here)
SLICE_MAX = 128        # slices per row preferred at 16 slots per lane
GROUPS_MAX = 8192      # workgroups of the first launch preferred at 16 slots per lane
MAX_SLICES = 1024      # hard limit of a split plan
BLOCKS = (64, 128, 256, 512, 1024)
PARAMS = ["a", "b", "e", "c", "d"]


def _slices(cols: int, block: int, slots: int) -> int:
    return -(-cols // (block * slots))


def slice_plan(op: str, rows: int, cols: int):
    """(block, slots) of the split plan the rule picks, or None when no split
    plan is legal (rows out of range, too few or too many slices, bfloat16
    rows whose length is not a multiple of 8)."""
    if rows < 1 or rows >= ROWS_LIMIT:
        return None
    if op.endswith("_bf16") and cols % 8 != 0:
        return None
    for block in BLOCKS:
        s = _slices(cols, block, 16)
        if 2 <= s <= SLICE_MAX and rows * s <= GROUPS_MAX:
            return block, 16
    s = _slices(cols, 1024, 32)
    if 2 <= s <= MAX_SLICES:
        return 1024, 32
    return None


def split_key(block: int, slots: int) -> str:
    return f"b{block}-k{slots}"


def predict(theta: dict, op: str, rows: int, cols: int) -> tuple[float, float]:
    """(plain, split) predicted microseconds per call."""
    a, b, e, c, d = theta[op]
    return a + b * cols + e * rows * cols, c + d * rows * cols


def choose(theta: dict, op: str, rows: int, cols: int) -> str:
    """"plain" or the split key the selector takes."""
    sp = slice_plan(op, rows, cols)
    if sp is None:
        return "plain"
    tp, ts = predict(theta, op, rows, cols)
    return split_key(*sp) if ts < tp else "plain"


# ---------------------------------------------------------------- data

TRAIN_COLS = (8192, 16384, 32768, 65536, 131072, 262144, 1 << 20)
TRAIN_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 255)
HELDOUT_COLS = (12288, 24576, 49152, 98304, 196608, 393216, 786432)
HELDOUT_ROWS = (3, 6, 12, 24, 48, 96, 192)
MAX_ELEMENTS = 1 << 25


def measure(out_json: str, ops: list[str], cols_list, rows_list) -> None:
    """GPU: per (op, rows, cols) with rows * cols <= MAX_ELEMENTS, the per-call
    time (graph-replayed, inputs cycled cold above 1 MiB as the plan search
    does) of the plan the plain entry point selects and of every legal split
    plan with 16 or 32 slots per lane; median of five samples."""
    import time
    import torch
    import row_reduction_amd as rr
    from row_reduction_amd import _capi
    from row_reduction_amd._capi import RR_PATH_SPLIT, rr_plan
    from row_reduction_amd.tune import Case, GraphTimer, launches_per_graph
    dev = torch.device("cuda:0")
    res, t0 = [], time.time()
    for op in ops:
        v = 8 if op.endswith("_bf16") else 4
        for cols in cols_list:
            for rows in rows_list:
                if rows * cols > MAX_ELEMENTS:
                    continue
                cands = [rr_plan(RR_PATH_SPLIT, b, b, 1, v, k, 2) for b in BLOCKS for k in (16, 32)]
                cands = [p for p in cands if rr.rr_check_plan(op, rows, cols, p) == _capi.RR_OK]
                plain = rr.rr_select_plan(op, rows, cols)
                case = Case(torch, op, rows, cols, False, dev, hot=False, workspace=False)
                case.ws = torch.empty(rows * MAX_SLICES * 16, dtype=torch.uint8, device=dev)
                us = {}
                for p in [plain] + cands:
                    key = "plain" if p.path != RR_PATH_SPLIT else split_key(p.block, p.slots)
                    gt = GraphTimer(torch, case, p, launches_per_graph(torch, case, p))
                    us[key] = round(sorted(gt.sample_us() for _ in range(5))[2], 3)
                    del gt
                res.append({"op": op, "rows": rows, "cols": cols, "cold": case.cold,
                            "plain_plan": plain.as_dict(), "us": us})
                print(f"{time.time() - t0:6.1f}s {op} {rows}x{cols} plain {us['plain']} us", flush=True)
                del case
                torch.cuda.empty_cache()
        with open(out_json, "w") as f:
            json.dump(res, f)


def export(out_csv: str, json_files: list[str]) -> int:
    """Grid timings (lists of {op, rows, cols, cold, us: {key: us}}) to CSV."""
    n = 0
    with open(out_csv, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["op", "rows", "cols", "cold", "plan", "us"])
        for path in json_files:
            for r in json.load(open(path)):
                for key, us in sorted(r["us"].items()):
                    w.writerow([r["op"], r["rows"], r["cols"], int(bool(r["cold"])), key, f"{us:.3f}"])
                    n += 1
    return n


def load(path: str = DATA) -> list[dict]:
    """Cases {op, rows, cols, cold, t: {plan key: us}} in file order."""
    cases, index = [], {}
    for r in csv.DictReader(open(path)):
        k = (r["op"], int(r["rows"]), int(r["cols"]))
        if k not in index:
            index[k] = len(cases)
            cases.append({"op": k[0], "rows": k[1], "cols": k[2], "cold": int(r["cold"]), "t": {}})
        cases[index[k]]["t"][r["plan"]] = float(r["us"])
    return cases


# ---------------------------------------------------------------- fit

def fit(cases: list[dict]) -> dict:
    """Per operator: (a, b, e) on the plain timings and (c, d) on the timings
    of the rule's split plan, each by least squares on relative error."""
    theta = {}
    for op in OPS:
        cs = [c for c in cases if c["op"] == op]
        if not cs:
            raise SystemExit(f"no timings for {op}")
        A = np.array([[1.0, c["cols"], c["rows"] * c["cols"]] for c in cs])
        y = np.array([c["t"]["plain"] for c in cs])
        abe = np.linalg.lstsq(A / y[:, None], np.ones(len(y)), rcond=None)[0]
        ss = [(c, split_key(*slice_plan(op, c["rows"], c["cols"]))) for c in cs
              if slice_plan(op, c["rows"], c["cols"]) is not None]
        ss = [(c, k) for c, k in ss if k in c["t"]]
        A = np.array([[1.0, c["rows"] * c["cols"]] for c, _ in ss])
        y = np.array([c["t"][k] for c, k in ss])
        cd = np.linalg.lstsq(A / y[:, None], np.ones(len(y)), rcond=None)[0]
        theta[op] = tuple(float(v) for v in (*abe, *cd))
    return theta


def regrets(cases: list[dict], chooser) -> list[float]:
    """Per case: time of the chosen plan / fastest timed plan - 1."""
    out = []
    for c in cases:
        k = chooser(c)
        if k not in c["t"]:
            k = "plain"
        out.append(c["t"][k] / min(c["t"].values()) - 1.0)
    return out


def old_rule(c: dict) -> str:
    """The selector's earlier fixed rule: split whenever rows < 256 and cols >=
    8192, 256 lanes x 16 slots per slice (widened while a row would need more
    than 1024 slices)."""
    rows, cols = c["rows"], c["cols"]
    if rows >= 256 or cols < 8192:
        return "plain"
    if c["op"].endswith("_bf16") and cols % 8 != 0:
        return "plain"
    for block, slots in ((256, 16), (256, 32), (1024, 32)):
        if 2 <= _slices(cols, block, slots) <= MAX_SLICES:
            return split_key(block, slots)
    return "plain"


def report(theta: dict, paths: list[str]) -> str:
    lines = ["| Timings | Cases | Selector | Mean regret | Median | Max | Cases > 10 % |",
             "|---|---:|---|---:|---:|---:|---:|"]
    for path in paths:
        cases = load(path)
        for name, fn in (("fitted split model", lambda c: choose(theta, c["op"], c["rows"], c["cols"])),
                         ("fixed rule (rows < 256, cols >= 8192)", old_rule),
                         ("never split", lambda c: "plain")):
            r = regrets(cases, fn)
            lines.append(f"| {os.path.basename(path)} | {len(r)} | {name} | {statistics.mean(r):.2%} | "
                         f"{statistics.median(r):.2%} | {max(r):.1%} | {sum(x > 0.10 for x in r)} |")
    return "\n".join(lines)


# ---------------------------------------------------------------- frozen constants

def emit(theta: dict, path: str = INC) -> None:
    lines = ["// Generated by row_reduction_amd/split_model.py --fit ... --emit: per operator",
             "// (rr_op order) the split-row selector's constants {a, b, e, c, d}, fitted to",
             "// the committed split/plain timings: plain us = a + b*cols + e*rows*cols,",
             "// split us = c + d*rows*cols."]
    for op in OPS:
        vals = ", ".join(repr(v) for v in theta[op])
        lines.append(f"{{{vals}}},  // {op}")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_inc(path: str = INC) -> dict:
    theta = {}
    for line in open(path):
        if line.startswith("{"):
            body, op = line.split("//")
            theta[op.strip()] = tuple(float(v) for v in body.strip().rstrip(",").strip("{}").split(","))
    return theta


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--measure", metavar="OUT_JSON", help="GPU: time plain and split plans over a grid")
    ap.add_argument("--ops", default=",".join(OPS))
    ap.add_argument("--cols", default=",".join(map(str, TRAIN_COLS)))
    ap.add_argument("--rows", default=",".join(map(str, TRAIN_ROWS)))
    ap.add_argument("--export", nargs="+", metavar=("OUT_CSV", "JSON"))
    ap.add_argument("--fit", metavar="CSV")
    ap.add_argument("--emit", action="store_true", help="write csrc/split_model.inc from --fit")
    ap.add_argument("--report", nargs="+", metavar="CSV", help="regret table of the frozen constants")
    a = ap.parse_args()
    if a.measure:
        measure(a.measure, [o for o in a.ops.split(",") if o], [int(c) for c in a.cols.split(",")],
                [int(r) for r in a.rows.split(",")])
        return 0
    if a.export:
        print(export(a.export[0], a.export[1:]), "rows")
        return 0
    if a.fit:
        theta = fit(load(a.fit))
        for op in OPS:
            print(op, theta[op])
        if a.emit:
            emit(theta)
            print("wrote", INC)
        return 0
    if a.report:
        print(report(read_inc(), a.report))
        return 0
    ap.print_help()
    return 1


if __name__ == "__main__":
    sys.exit(main())

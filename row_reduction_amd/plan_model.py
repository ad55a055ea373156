"""Analytic launch-plan cost model: the plan selector for (operator, shape)
pairs the measured table does not list.

The LuisaCompute notes ("Consecutive-worker reduction layout checkpoint",
section "Evidence and what remains") observe that a scalar per-round cost
prior could not rank layouts because it ignored how many workgroups stay
active once rows are packed and what the pack width does to issue and memory
behaviour; the MPP memory notes price occupancy with a waves term. This model
prices exactly those effects for one launch on a 256-CU gfx950 part, from the
plan's integers alone:

  * memory:   algorithmic bytes (plus a fraction of the streaming path's
              re-read bytes) over an effective bandwidth that saturates with
              the bytes the resident lanes keep in flight (Little's law:
              in-flight bytes / latency, capped at the HBM rate), reduced
              when one wave load instruction covers only a short contiguous
              run of a row (narrow packs, rows shared by few lanes);
  * latency:  per round of resident workgroups, a chain of wave start-up,
              per-lane loads and stores, per-element ALU work, the
              cross-lane reduction steps and, on the streaming path, a fixed
              loop cost;
  * issue:    total lane-instructions of all waves over the chip, divided by
              the waves each SIMD keeps resident (occupancy from a register
              estimate);
  * dispatch: a cost per wave and per workgroup launched;

combined as a smooth maximum (4-norm) on top of the measured launch floor. Constants
are fitted once (least squares on log time, each case's mean removed so only
the ranking inside a case is fitted) to the committed timings of the plan
search, and frozen into csrc/plan_model.inc; the C++ planner evaluates the
same formulas (rr_model_time_us) and picks the cheapest legal candidate.

  python -m row_reduction_amd.plan_model --export OUT.csv search.json [train/*.json ...]
  python -m row_reduction_amd.plan_model --fit row_reduction_amd/data/plan_timings.csv --emit
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import os
import re
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DATA = os.path.join(HERE, "data", "plan_timings.csv")
INC = os.path.join(HERE, "csrc", "plan_model.inc")

# Per operator: row arrays read, row arrays written, weight arrays, ALU
# operations per element, registers per kept slot, passes on the streaming path.
OPS = {
    "rmsnorm": (1, 1, 1, 4, 2.4, 2),
    "sum": (1, 0, 0, 3, 2.0, 1),
    "softmax": (1, 1, 0, 9, 1.6, 2),
    "layernorm": (1, 1, 2, 8, 3.2, 2),
    "residual_layernorm": (2, 2, 2, 10, 3.3, 2),
    "cross_entropy": (1, 0, 0, 7, 1.6, 1),
}
PATHS = {"packed": 0, "row": 1, "loop": 2}
NCU = 256                      # compute units
FLOOR_US = 1.59               # measured interval between back-to-back empty launches
PARAMS = ["bw_gbps", "lat_us", "reread", "run_bytes", "wave_us", "group_us",
          "chain_us", "chain_wave_us", "chain_mem_us", "chain_elem_us", "chain_red_us",
          "issue_us", "loop_mem_us", "loop_us"]
P0 = [6500.0, 0.5, 0.4, 64.0, 1e-4, 1e-4, 0.3, 0.05, 0.01, 5e-4, 0.03, 5e-5, 0.05, 0.3]
LO = [3000, 0.05, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0]
HI = [8000, 10, 1.5, 4096, 1e-2, 1e-2, 5, 1, 1, 0.1, 1, 1e-2, 2, 3]


def parse_key(key: str) -> dict:
    m = re.match(r"(packed|row|loop)-b(\d+)-w(\d+)-v(\d+)-k(\d+)-c(\d)", key)
    b, w, v, k, c = map(int, m.groups()[1:])
    return {"path": PATHS[m.group(1)], "block": b, "lanes": w, "v": v, "slots": k, "cache": c}


def lds_slots(base: str, bf: bool, p: dict) -> int:
    """Values per lane a streaming plan also keeps in LDS between its passes,
    as the kernels do (1024-lane groups only): the LayerNorms at 32 register
    slots and softmax at 64 keep 32 floats per lane, or 72 bfloat16 values
    for bfloat16 rows; softmax at 96 keeps 32; bfloat16 RMSNorm at 64 slots
    with v = 8 keeps 72."""
    B, V, K = p["block"], p["v"], p["slots"]
    if p["path"] != 2 or B != 1024 or K == 0:
        return 0
    if K == 96 and base == "softmax":
        return 32
    if (K == 32 and base in ("layernorm", "residual_layernorm")) or (K == 64 and base == "softmax"):
        return 72 if bf else 32
    if bf and V == 8 and K == 64 and base == "rmsnorm":
        return 72
    return 0


def features(op: str, rows: int, cols: int, p: dict) -> dict:
    """Integer-derived quantities of one launch (all paths of the model)."""
    bf = op.endswith("_bf16")
    base = op[:-5] if bf else op
    E = 2 if bf else 4
    n_in, n_out, n_w, alu, vps, passes = OPS[base]
    path, B, W, V, K = p["path"], p["block"], p["lanes"], p["v"], p["slots"]
    R = B // W
    G = -(-rows // R)
    nw = B // 64
    if path == 2:
        nch = -(-cols // (W * V))
        held = K + lds_slots(base, bf, p)
        kept_cols = min(cols, W * held)
        vgpr = 24 + 1.2 * K + 2 * V
        loads = nch * (n_in * passes + n_w) - min(held // V, nch) * n_in * (passes - 1)
        elems = nch * V * passes
        exact = False
    else:
        nch = K // V
        kept_cols = cols
        vgpr = 16 + vps * K
        loads = nch * (n_in + n_w)
        elems = K
        exact = W * K == cols
    occ = min(8, 512 // (8 * math.ceil(vgpr / 8)))
    groups_cu = max(1, min(32, (4 * occ) // nw))
    cap = NCU * groups_cu
    active = min(G, cap)
    nbytes = rows * cols * E * (n_in + n_out) + (rows * 4 if n_out == 0 else 0)
    reread = rows * E * n_in * max(0, cols - kept_cols) if (path == 2 and passes == 2) else 0
    per_lane = (V if path == 2 else K) * E * n_in
    nred = 1 if base in ("sum", "rmsnorm") else 2
    red = nred * (2 * math.log2(min(W, 64)) + (4 if W > 64 else 0))
    run = min(W, 64) * V * E   # contiguous bytes of one row per wave load instruction
    return {"bytes": float(nbytes), "reread": float(reread), "inflight": float(active * B * per_lane),
            "run": float(run),
            "rounds": float(-(-G // cap)), "loads": float(loads), "stores": float(nch * n_out),
            "elems": float(elems * (alu + (0 if exact else 2))), "red": float(red), "waves": float(G * nw),
            "groups": float(G), "nw": float(nw), "occ": float(occ), "path": float(path)}


def _p4(x):
    y = x * x
    return y * y


def predict_us(f, th):
    """Predicted microseconds per launch; f holds scalars or equal-length arrays."""
    (bw, lat, reread, run_bytes, wave_us, group_us, chain_us, chain_wave_us, chain_mem_us,
     chain_elem_us, chain_red_us, issue_us, loop_mem_us, loop_us) = th
    xp = np if isinstance(f["path"], np.ndarray) else math
    loop = f["path"] == 2
    bw_lat = f["inflight"] / lat / 1e3
    # Smooth minimum of the HBM rate and the latency-bound rate (4-norm of
    # reciprocals), written with products and square roots only.
    inv4 = 1.0 / _p4(bw) + 1.0 / _p4(bw_lat)
    bw_eff = 1.0 / xp.sqrt(xp.sqrt(inv4)) / (1.0 + run_bytes / f["run"])
    t_mem = (f["bytes"] + reread * f["reread"]) / (bw_eff * 1e3)
    mem_ops = f["loads"] + f["stores"]
    t_group = (chain_us + chain_wave_us * f["nw"] + chain_mem_us * mem_ops + chain_elem_us * f["elems"]
               + chain_red_us * f["red"])
    t_group = t_group + (np.where(loop, loop_mem_us * f["loads"] + loop_us, 0.0) if xp is np else
                         (loop_mem_us * f["loads"] + loop_us if loop else 0.0))
    t_chain = f["rounds"] * t_group
    t_issue = issue_us * f["waves"] * (mem_ops + 0.25 * f["elems"] + f["red"])
    t_disp = wave_us * f["waves"] + group_us * f["groups"]
    return FLOOR_US + xp.sqrt(xp.sqrt(_p4(t_mem) + _p4(t_chain) + _p4(t_issue) + _p4(t_disp)))


# ---- data ----------------------------------------------------------------------

def export(out_csv: str, paths: list[str]) -> int:
    """Timings of the plan search (tune.py output) as CSV rows, keeping per
    case the cache policy the selector would use (2 when timed cold, else 0)."""
    n = 0
    with open(out_csv, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["op", "rows", "cols", "cold", "plan", "us"])
        for path in paths:
            for c in json.load(open(path))["cases"]:
                want = 2 if c["cold"] else 0
                for key, r in sorted(c["candidates"].items()):
                    if "us" in r and parse_key(key)["cache"] == want:
                        wr.writerow([c["op"], c["rows"], c["cols"], int(c["cold"]), key, "%.4f" % r["us"]])
                        n += 1
    return n


def load(csv_path: str = DATA):
    rows = list(csv.DictReader(open(csv_path)))
    cases, idx = [], {}
    for r in rows:
        k = (r["op"], int(r["rows"]), int(r["cols"]))
        if k not in idx:
            idx[k] = len(cases)
            cases.append({"op": k[0], "rows": k[1], "cols": k[2], "t": {}})
        cases[idx[k]]["t"][r["plan"]] = float(r["us"])
    return cases


def arrays(cases):
    feats, t, case = [], [], []
    for ci, c in enumerate(cases):
        for key, us in c["t"].items():
            feats.append(features(c["op"], c["rows"], c["cols"], parse_key(key)))
            t.append(us)
            case.append(ci)
    F = {k: np.array([f[k] for f in feats]) for k in feats[0]}
    return F, np.array(t), np.array(case)


def fit(cases):
    from scipy.optimize import least_squares
    F, t, case = arrays(cases)
    logt = np.log(t)
    cnt = np.bincount(case)

    def resid(th):
        e = np.log(predict_us(F, th)) - logt
        return e - (np.bincount(case, weights=e) / cnt)[case]

    r = least_squares(resid, P0, bounds=(LO, HI), loss="soft_l1", f_scale=0.05, max_nfev=3000, x_scale="jac")
    return list(r.x)


def regrets(cases, th):
    """Per case: measured time of the model's pick over the case's best, minus 1."""
    F, t, case = arrays(cases)
    pred = predict_us(F, th)
    out = []
    for ci in range(len(cases)):
        m = case == ci
        i = np.flatnonzero(m)[np.argmin(pred[m])]
        out.append(t[i] / t[m].min() - 1.0)
    return np.array(out)


def emit(th, path: str = INC) -> None:
    lines = ["// Generated by row_reduction_amd/plan_model.py --fit ... --emit: constants of the",
             "// analytic plan cost model, fitted to the committed plan-search timings.",
             "// Order: " + ", ".join(PARAMS) + "."]
    lines += ["%.17g," % x for x in th]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def read_inc(path: str = INC) -> list[float]:
    vals = [float(l.strip().rstrip(",")) for l in open(path) if l.strip() and not l.startswith("//")]
    assert len(vals) == len(PARAMS)
    return vals


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--export", nargs="+", metavar=("OUT_CSV", "SEARCH_JSON"))
    ap.add_argument("--fit", metavar="CSV")
    ap.add_argument("--emit", action="store_true", help="write csrc/plan_model.inc")
    args = ap.parse_args()
    if args.export:
        print(export(args.export[0], args.export[1:]), "rows")
        return 0
    if args.fit:
        cases = load(args.fit)
        th = fit(cases)
        rg = regrets(cases, th)
        print(json.dumps(dict(zip(PARAMS, th)), indent=1))
        print("in-sample regret: mean %.4f median %.4f max %.4f, > 10%%: %d of %d"
              % (rg.mean(), np.median(rg), rg.max(), int((rg > 0.1).sum()), len(rg)))
        if args.emit:
            emit(th)
        return 0
    ap.print_help()
    return 1


if __name__ == "__main__":
    sys.exit(main())

"""Offline plan search: per (operator, shape), time every legal plan on the
GPU and freeze the fastest into the library's plan table.

Protocol, after the LuisaCompute notes "Consecutive-worker reduction layout
checkpoint" (sections "Evidence and what remains" and "Measurement
contract"):
  * a finite candidate grid (plans.candidate_plans) filtered by the library's
    legality check before anything is timed;
  * the objective is GPU time: each sample is one replay of a HIP graph
    holding `n` back-to-back launches, timed with HIP events, divided by n
    (the graph removes host launch cost, like the pages' command-buffer
    interval divided by batch size); a candidate whose launch fails or whose
    output disagrees with the rule plan's output is rejected;
  * search: several rounds with the candidate order rotated each round;
    table value = median of per-round medians;
  * replay (`--replay`): a fresh process on a held-out seed re-measures the
    winner against the incumbent plan in position-balanced A/B order; a
    winner enters the table only if the replay measures it at least
    MIN_GAIN (1 %) faster.

Shapes whose working set would stay in the 256 MB last-level cache are timed
cold: each graph cycles over enough distinct input/output buffers (>= 768 MiB)
that no launch finds its data cached.

Usage:
  python -m row_reduction_amd.tune --out search.json [--ops rmsnorm,...] [--shapes 1x127,...]
                                   [--caches all|by-footprint|0,2]
  python -m row_reduction_amd.tune --replay search.json --out replay.json
  python -m row_reduction_amd.tune --emit-table replay.json   # writes csrc/plan_table.inc
  python -m row_reduction_amd.tune --summarize search.json replay.json
  python -m row_reduction_amd.tune --validate --heldout 30 --out validate.json
  python -m row_reduction_amd.tune --summarize-validate validate.json
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from row_reduction_amd import _capi, plans, workloads  # noqa: E402
from row_reduction_amd._capi import rr_plan  # noqa: E402

COLD_BYTES = 768 << 20
# A search winner replaces the incumbent plan only when the held-out replay
# measures it at least this much faster (paired median), so that run-to-run
# noise does not churn the table.
MIN_GAIN = 0.01
GRAPH_TARGET_US = 2000.0
DEFAULT_SHAPES = ["1x127", "17x257", "64x4096", "1024x4096", "16384x8192"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    """sha256 over the device sources (what the timings depend on)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in ("device.h", "internal.h") or name.startswith("kernels_"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def host_inputs(op: str, rows: int, cols: int, held_out: bool) -> dict:
    """Seeded inputs with the measured configurations' distributions (bfloat16
    operators: the same draws as bfloat16 bit patterns)."""
    if op.endswith("_bf16"):
        d = host_inputs(op[:-5], rows, cols, held_out)
        return {k: (workloads.as_bf16_bits(v) if isinstance(v, np.ndarray) and v.dtype == np.float32
                    else v) for k, v in d.items()}
    if op == "rmsnorm":
        k = {(1, 127): 1, (17, 257): 2, (64, 4096): 3}.get((rows, cols), 4)
        seed = (2000 if held_out else 1000) + k
        wl = workloads.rmsnorm_workload(rows, cols, seed, outlier_fraction=0.01 if k == 3 else 0.0)
        return {"x": wl.x, "w": wl.w, "eps": wl.eps}
    seed = (2000 if held_out else 1000) + 5
    d = workloads.family_inputs(rows, cols, seed)
    return {"x": d["x"], "w": d["gamma"], "beta": d["beta"], "residual": d["residual"],
            "targets": d["targets"], "eps": workloads.LAYERNORM_EPS}


class Case:
    """Device buffers for one (op, shape), replicated into enough sets to run cold."""

    def __init__(self, torch, op, rows, cols, held_out, device, hot=False, workspace=False):
        import row_reduction_amd as rr
        self.torch, self.rr, self.op, self.rows, self.cols = torch, rr, op, rows, cols
        h = host_inputs(op, rows, cols, held_out)
        self.host = h  # the seeded host arrays every buffer set is a copy of
        self.eps = h["eps"]
        self.bf16 = op.endswith("_bf16")
        self.base = op[:-5] if self.bf16 else op

        def dev_tensor(v):
            if v.dtype == np.uint16:
                return torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
            return torch.from_numpy(v).to(device)
        dev = {k: dev_tensor(v) for k, v in h.items() if k != "eps"}
        elem = 2 if self.bf16 else 4
        per_set = elem * rows * cols * (3 if self.base == "residual_layernorm" else 2)
        # Cold: enough distinct sets that the cycled footprint is >= COLD_BYTES,
        # three times the 256 MB last-level cache, so no launch finds its data
        # there. A single set of COLD_BYTES or more is cold by itself.
        self.nsets = 1
        if not hot and per_set >= (1 << 20):
            self.nsets = int(min(1024, -(-COLD_BYTES // per_set)))
        self.cold = self.nsets > 1 or per_set >= COLD_BYTES
        self.cold_possible = per_set >= (1 << 20)
        # Optional split-row workspace (shared by the sets: launches are sequential).
        self.ws = None
        if workspace:
            n = rr.rr_workspace_bytes(op, rows, cols)
            if n > 0:
                self.ws = torch.empty(n, dtype=torch.uint8, device=device)
        self.sets = []
        for _ in range(self.nsets):
            s = dict(dev)
            s["x"] = dev["x"].clone()
            if self.base == "residual_layernorm":
                s["residual"] = dev["residual"].clone()
            if self.base in ("sum", "cross_entropy"):
                s["out"] = torch.empty(rows, dtype=torch.float32, device=device)
            else:
                s["out"] = torch.empty_like(dev["x"])
            self.sets.append(s)

    def launch(self, i: int, plan) -> None:
        s, rr = self.sets[i % self.nsets], self.rr
        op, sfx = self.base, ("_bf16" if self.bf16 else "_f32")
        kw = {"plan": plan, "workspace": self.ws}
        if op == "rmsnorm":
            getattr(rr, "rmsnorm" + sfx)(s["x"], s["w"], self.eps, y=s["out"], **kw)
        elif op == "sum":
            getattr(rr, "row_sum" + sfx)(s["x"], out=s["out"], **kw)
        elif op == "softmax":
            getattr(rr, "softmax" + sfx)(s["x"], y=s["out"], **kw)
        elif op == "layernorm":
            getattr(rr, "layernorm" + sfx)(s["x"], s["w"], s["beta"], self.eps, y=s["out"], **kw)
        elif op == "residual_layernorm":
            getattr(rr, "residual_layernorm" + sfx)(s["x"], s["residual"], s["w"], s["beta"], self.eps,
                                                    y=s["out"], **kw)
        elif op == "cross_entropy":
            getattr(rr, "cross_entropy" + sfx)(s["x"], s["targets"], loss=s["out"], **kw)

    def output(self):
        return self.sets[0]["out"]


class GraphTimer:
    """A HIP graph of n launches of one plan, replayed and timed with events."""

    def __init__(self, torch, case: Case, plan, n: int):
        self.torch = torch
        case.launch(0, plan)                      # eager once: errors surface here
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(n):
                case.launch(i, plan)
        self.n = n
        self.start = torch.cuda.Event(enable_timing=True)
        self.stop = torch.cuda.Event(enable_timing=True)
        self.graph.replay()
        torch.cuda.synchronize()

    def sample_us(self) -> float:
        self.start.record()
        self.graph.replay()
        self.stop.record()
        self.stop.synchronize()
        return self.start.elapsed_time(self.stop) * 1000.0 / self.n


def launches_per_graph(torch, case: Case, plan) -> int:
    t = torch.cuda.Event(enable_timing=True)
    u = torch.cuda.Event(enable_timing=True)
    case.launch(0, plan)
    torch.cuda.synchronize()
    t.record()
    for i in range(5):
        case.launch(i, plan)
    u.record()
    u.synchronize()
    per = max(t.elapsed_time(u) * 1000.0 / 5, 1.0)
    n = int(GRAPH_TARGET_US / per)
    n = max(case.nsets, min(400, max(8, n)))
    if case.nsets > 1:
        n = max(case.nsets, (n // case.nsets) * case.nsets)
    return n


def close(a, b) -> bool:
    """Outputs of two plans agree: float within 2e-5 relative, bfloat16 within
    one unit in the last place (2^-7 relative)."""
    rel = 2.0 ** -7 if a.dtype != b.dtype or str(a.dtype) == "torch.bfloat16" else 2e-5
    a = a.double()
    b = b.double()
    return bool(((a - b).abs() <= 2e-5 + rel * b.abs()).all().item())


def measure(torch, case: Case, candidates: dict, rounds: int, samples: int) -> dict:
    """Median-of-round-medians us/op for each candidate; rotated order per round."""
    import row_reduction_amd as rr
    ref_plan = rr.rr_select_plan(case.op, case.rows, case.cols)
    case.launch(0, ref_plan)
    torch.cuda.synchronize()
    ref_out = case.output().clone()
    timers, results = {}, {}
    n = None
    for key, p in candidates.items():
        try:
            if n is None:
                n = launches_per_graph(torch, case, p)
            timers[key] = GraphTimer(torch, case, p, n)
            if not close(case.output(), ref_out):
                results[key] = {"plan": p.as_dict(), "rejected": "output differs from rule plan"}
                del timers[key]
        except Exception as e:  # a failed launch rejects the candidate
            results[key] = {"plan": p.as_dict(), "rejected": f"{type(e).__name__}: {e}"}
            timers.pop(key, None)
    keys = list(timers)
    raw = {k: [] for k in keys}
    for r in range(rounds):
        order = keys[r % max(1, len(keys)):] + keys[:r % max(1, len(keys))]
        if r % 2 == 1:
            order = order[::-1]
        for k in order:
            raw[k].append([timers[k].sample_us() for _ in range(samples)])
    nbytes = workloads.algorithmic_bytes(case.op, case.rows, case.cols)
    for k in keys:
        med = statistics.median(statistics.median(rs) for rs in raw[k])
        flat = [v for rs in raw[k] for v in rs]
        results[k] = {"plan": candidates[k].as_dict(), "us": med, "min_us": min(flat),
                      "max_us": max(flat), "GBps": nbytes / (med * 1e3), "raw_us": raw[k]}
    del timers
    return results


def run_search(args) -> dict:
    import torch
    import row_reduction_amd as rr
    _capi.lib()
    device = torch.device("cuda:0")
    out = {"kind": "search", "source_sha256": source_hash(), "rounds": args.rounds,
           "samples": args.samples, "cases": []}
    for op in args.ops:
        for shape in args.shapes:
            rows, cols = map(int, shape.split("x"))
            log(f"search {op} {shape}")
            case = Case(torch, op, rows, cols, False, device)
            caches = plans.CACHES
            if args.caches == "by-footprint":
                # One policy per case: non-temporal row data when the working
                # set is timed cold, default caching when it stays resident.
                caches = (2,) if case.cold else (0,)
            elif args.caches != "all":
                caches = tuple(int(c) for c in args.caches.split(","))
            cands = {plans.plan_key(p): p for p in plans.candidate_plans(op, rows, cols, caches=caches)}
            res = measure(torch, case, cands, args.rounds, args.samples)
            timed = {k: v for k, v in res.items() if "us" in v}
            best = min(timed, key=lambda k: timed[k]["us"])
            rule = plans.plan_key(rr.rr_select_plan(op, rows, cols))
            out["cases"].append({"op": op, "rows": rows, "cols": cols, "cold": case.cold,
                                 "nsets": case.nsets, "winner": best, "rule": rule,
                                 "candidates": res})
            log(f"  winner {best} {timed[best]['us']:.3f} us ({timed[best]['GBps']:.0f} GB/s); "
                f"rule {rule} {timed.get(rule, {}).get('us', float('nan')):.3f} us")
            del case
            torch.cuda.empty_cache()
    return out


def heldout_shapes(n: int, seed: int) -> list[str]:
    """n seeded (rows, cols) drawn log-uniformly (rows 1..65536, cols
    32..32768, at most 2^27 elements), none of them a shape the plan table or
    the model's training timings list."""
    import random
    rnd = random.Random(seed)
    taken = set()
    for path in (os.path.join(HERE, "data", "plan_timings.csv"),):
        if os.path.exists(path):
            import csv
            taken |= {(int(r["rows"]), int(r["cols"])) for r in csv.DictReader(open(path))}
    out = []
    while len(out) < n:
        rows = int(round(2 ** rnd.uniform(0, 16)))
        cols = int(round(2 ** rnd.uniform(5, 15)))
        if rows * cols <= (1 << 27) and (rows, cols) not in taken:
            taken.add((rows, cols))
            out.append(f"{rows}x{cols}")
    return out


def run_validate(args) -> dict:
    """Held-out check of the plan sources: per case, every candidate at the
    footprint's cache policy plus the exact plans of the analytic model and
    of the built-in rule, timed together; regret = chosen time / best - 1."""
    import torch
    import row_reduction_amd as rr
    _capi.lib()
    device = torch.device("cuda:0")
    out = {"kind": "validate", "source_sha256": source_hash(), "rounds": args.rounds,
           "samples": args.samples, "cases": []}
    for op in args.ops:
        for shape in args.shapes:
            rows, cols = map(int, shape.split("x"))
            log(f"validate {op} {shape}")
            case = Case(torch, op, rows, cols, False, device)
            caches = (2,) if case.cold else (0,)
            cands = {plans.plan_key(p): p for p in plans.candidate_plans(op, rows, cols, caches=caches)}
            chosen = {src: rr.rr_select_plan_from(op, rows, cols, src) for src in ("model", "rule")}
            for p in chosen.values():
                cands.setdefault(plans.plan_key(p), p)
            res = measure(torch, case, cands, args.rounds, args.samples)
            timed = {k: v["us"] for k, v in res.items() if "us" in v}
            best = min(timed, key=timed.get)
            entry = {"op": op, "rows": rows, "cols": cols, "cold": case.cold, "best": best,
                     "best_us": timed[best], "candidates": {k: round(v, 4) for k, v in timed.items()}}
            for src, p in chosen.items():
                k = plans.plan_key(p)
                entry[src] = k
                entry[src + "_us"] = timed.get(k)
                entry[src + "_regret"] = timed[k] / timed[best] - 1.0 if k in timed else None
            out["cases"].append(entry)
            log(f"  best {best} {timed[best]:.3f} us; model {entry['model']} regret "
                f"{entry['model_regret']}; rule {entry['rule']} regret {entry['rule_regret']}")
            del case
            torch.cuda.empty_cache()
    return out


def summarize_validate(path: str) -> str:
    v = json.load(open(path))
    cs = [c for c in v["cases"] if c.get("model_regret") is not None and c.get("rule_regret") is not None]
    out = [f"Device source sha256: `{v['source_sha256']}`; {v['rounds']} rounds x {v['samples']} samples; "
           f"{len(cs)} held-out (operator, shape) cases.", ""]

    def stats(key):
        r = sorted(c[key] for c in cs)
        return (statistics.mean(r), statistics.median(r), r[-1], sum(1 for x in r if x > 0.10),
                sum(1 for x in r if x <= 0.02))
    out.append("| Plan source | Mean regret | Median | Max | Cases > 10% | Cases within 2% |")
    out.append("|---|---:|---:|---:|---:|---:|")
    for src in ("model", "rule"):
        m, med, mx, over, near = stats(src + "_regret")
        out.append(f"| {src} | {m:.2%} | {med:.2%} | {mx:.1%} | {over} | {near} |")
    wins = sum(1 for c in cs if c["model_us"] < c["rule_us"] * 0.98)
    losses = sum(1 for c in cs if c["rule_us"] < c["model_us"] * 0.98)
    out += ["", f"Model faster than the rule by > 2%: {wins} cases; rule faster by > 2%: {losses}.", ""]
    out.append("| Op | Shape | Cache | Best (us) | Model plan (regret) | Rule plan (regret) |")
    out.append("|---|---|---|---|---|---|")
    for c in sorted(cs, key=lambda c: (c["op"], c["rows"] * c["cols"])):
        out.append(f"| {c['op']} | {c['rows']}x{c['cols']} | {'cold' if c['cold'] else 'hot'} | "
                   f"`{c['best']}` {c['best_us']:.2f} | `{c['model']}` {c['model_regret']:.1%} | "
                   f"`{c['rule']}` {c['rule_regret']:.1%} |")
    return "\n".join(out)


def run_replay(args) -> dict:
    import torch
    import row_reduction_amd as rr
    _capi.lib()
    device = torch.device("cuda:0")
    search = json.load(open(args.replay))
    out = {"kind": "replay", "source_sha256": source_hash(), "search_source_sha256":
           search["source_sha256"], "rounds": args.rounds, "samples": args.samples, "cases": []}
    if search["source_sha256"] != out["source_sha256"]:
        raise SystemExit("kernel sources changed since the search; run the search again")
    for c in search["cases"]:
        op, rows, cols = c["op"], c["rows"], c["cols"]
        win, rule = c["winner"], c["rule"]
        log(f"replay {op} {rows}x{cols}: {win} vs {rule}")
        case = Case(torch, op, rows, cols, True, device)
        cands = {win: rr_plan.from_dict(c["candidates"][win]["plan"])}
        if rule != win:
            cands[rule] = rr.rr_select_plan(op, rows, cols)
        res = measure(torch, case, cands, args.rounds, args.samples)
        entry = {"op": op, "rows": rows, "cols": cols, "winner": win, "rule": rule,
                 "cold": case.cold, "results": res}
        if rule != win and "us" in res.get(win, {}) and "us" in res.get(rule, {}):
            ratios = [statistics.median(b) / statistics.median(a)
                      for a, b in zip(res[win]["raw_us"], res[rule]["raw_us"])]
            entry["paired_speedup_median"] = statistics.median(ratios)
            entry["paired_speedup_range"] = [min(ratios), max(ratios)]
            entry["confirmed"] = statistics.median(ratios) >= 1.0 + MIN_GAIN
        else:
            entry["confirmed"] = rule == win
        out["cases"].append(entry)
        log(f"  confirmed={entry['confirmed']} speedup={entry.get('paired_speedup_median')}")
        del case
        torch.cuda.empty_cache()
    return out


def emit_table(path: str) -> str:
    """Write csrc/plan_table.inc from a replay file's confirmed winners."""
    rep = json.load(open(path))
    if rep.get("kind") != "replay":
        raise SystemExit("--emit-table takes a replay result")
    if rep["source_sha256"] != source_hash():
        raise SystemExit("kernel sources changed since the replay; measure again")
    lines = ["// Measured per-shape plans: {op, rows, cols, {path, block, lanes_per_row, rows_per_group, v, slots, cache}},",
             "// generated by row_reduction_amd/tune.py: the fastest legal plan of a GPU search on",
             "// MI355X, re-measured against the incumbent plan on held-out inputs in a",
             "// fresh process. [xxxxxxxx] on each line is the start of the sha256 of the device",
             "// sources it was measured under. Every measured shape is listed, so the table does",
             "// not depend on the built-in rule."]
    for c in rep["cases"]:
        # An unconfirmed winner leaves the incumbent (the plan selected when
        # the search ran) in place: the replay did not show it MIN_GAIN faster.
        if c["winner"] != c["rule"] and "paired_speedup_median" in c:
            c["confirmed"] = c["paired_speedup_median"] >= 1.0 + MIN_GAIN
        key = c["winner"] if c.get("confirmed") else c["rule"]
        if key not in c["results"] or "us" not in c["results"][key]:
            continue
        p = c["results"][key]["plan"]
        r = c["results"][key]
        lines.append(f"{{{_capi.OP_IDS[c['op']]}, {c['rows']}, {c['cols']}, {{{p['path']}, {p['block']}, "
                     f"{p['lanes_per_row']}, {p['rows_per_group']}, {p['v']}, {p['slots']}, "
                     f"{p.get('cache', 0)}}}}},  "
                     f"// [{rep['source_sha256'][:8]}] {c['op']} {c['rows']}x{c['cols']}: {r['us']:.3f} us"
                     + (f", x{c.get('paired_speedup_median', 1.0):.3f} vs incumbent" if c.get("confirmed")
                        else ", incumbent kept"))
    # Entries of the existing table for (op, rows, cols) this replay did not
    # measure are kept, with the device-source hash they were measured under.
    target = os.path.join(HERE, "csrc", "plan_table.inc")
    measured = {(_capi.OP_IDS[c["op"]], c["rows"], c["cols"]) for c in rep["cases"]}
    kept = []
    if os.path.exists(target):
        for line in open(target):
            if line.startswith("{"):
                head = line[1:].split(",")
                key = (int(head[0]), int(head[1]), int(head[2]))
                if key not in measured:
                    kept.append(line.rstrip("\n"))
    lines += kept
    with open(target, "w") as f:
        f.write("\n".join(lines) + "\n")
    return target


def summarize(search_path: str, replay_path: str) -> str:
    """Markdown summary of a search and its replay: per (op, shape) the number
    of legal candidates, the three fastest, the incumbent, and the replay."""
    search = json.load(open(search_path))
    replay = {(c["op"], c["rows"], c["cols"]): c for c in json.load(open(replay_path))["cases"]}
    out = [f"Device source sha256: `{search['source_sha256']}`; search {search['rounds']} rounds x "
           f"{search['samples']} samples, replay on held-out inputs.", "",
           "| Op | Shape | Cache | Legal plans | Fastest three (us per call) | Incumbent (us) | "
           "Replay: chosen vs incumbent, paired speedup [range] |",
           "|---|---|---|---:|---|---|---|"]
    for c in search["cases"]:
        timed = sorted(((k, v) for k, v in c["candidates"].items() if "us" in v), key=lambda kv: kv[1]["us"])
        top = "; ".join(f"`{k}` {v['us']:.3f}" for k, v in timed[:3])
        inc = c["candidates"].get(c["rule"], {})
        r = replay.get((c["op"], c["rows"], c["cols"]), {})
        if r.get("paired_speedup_median"):
            r["confirmed"] = r["paired_speedup_median"] >= 1.0 + MIN_GAIN
            rep = (f"{r['paired_speedup_median']:.3f} [{r['paired_speedup_range'][0]:.3f}, "
                   f"{r['paired_speedup_range'][1]:.3f}]" + ("" if r.get("confirmed") else " — not confirmed, incumbent kept"))
        else:
            rep = "winner is the incumbent"
        out.append(f"| {c['op']} | {c['rows']}x{c['cols']} | {'cold' if c['cold'] else 'hot'} | "
                   f"{len(timed)} | {top} | `{c['rule']}` {inc.get('us', float('nan')):.3f} | {rep} |")
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--ops", default=",".join(list(workloads.OPS) + [o + "_bf16" for o in workloads.OPS]))
    ap.add_argument("--shapes", default=",".join(DEFAULT_SHAPES))
    ap.add_argument("--rounds", type=int, default=2)
    ap.add_argument("--samples", type=int, default=5)
    ap.add_argument("--caches", default="all",
                    help="cache policies searched: all, by-footprint (2 when timed cold, else 0), or a list")
    ap.add_argument("--replay", help="search result to re-measure on held-out inputs")
    ap.add_argument("--emit-table", help="replay result to freeze into plan_table.inc")
    ap.add_argument("--summarize", nargs=2, metavar=("SEARCH", "REPLAY"),
                    help="print a markdown summary of a search and its replay")
    ap.add_argument("--validate", action="store_true",
                    help="time every candidate plus the model's and the rule's plans on held-out shapes")
    ap.add_argument("--heldout", type=int, metavar="N", help="use N seeded held-out shapes")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--summarize-validate", metavar="VALIDATE_JSON")
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.summarize:
        print(summarize(*args.summarize))
        return 0
    if args.summarize_validate:
        print(summarize_validate(args.summarize_validate))
        return 0
    args.ops = [o for o in args.ops.split(",") if o]
    args.shapes = [s for s in args.shapes.split(",") if s]
    if args.heldout:
        args.shapes = heldout_shapes(args.heldout, args.seed)
    if args.emit_table:
        print(emit_table(args.emit_table))
        return 0
    t0 = time.time()
    res = run_replay(args) if args.replay else (run_validate(args) if args.validate else run_search(args))
    res["elapsed_s"] = time.time() - t0
    text = json.dumps(res)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())

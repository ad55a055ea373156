"""Seeded random shapes for every operator and storage type, run with the
plan the library selects (table, else the analytic model), with and without
a split-row workspace, each compared element by element with the CPU
oracle. The fixed parity matrix names its plans; this covers whatever the
selector picks across the shape space."""
import os
import time

import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import plans, workloads

from parity_util import announce, compare, family_host_inputs, run_oracle, to_dev
from test_gpu_batch import rename
from test_gpu_bf16 import compare as compare_bf16
from test_gpu_bf16 import dev_inputs as dev_inputs_bf16
from test_gpu_bf16 import run_oracle as run_oracle_bf16
from test_gpu_split import IN_PLACE_OPS, run_bf16, run_f32, run_in_place

pytestmark = pytest.mark.gpu

OPS = list(workloads.OPS)


def shapes(seed, n, max_elems=1 << 22):
    """n (rows, cols) drawn log-uniformly, at most max_elems elements: every
    third draw a long row (cols 32768..140000, the streaming and split
    paths), the others rows 1..20000 and cols 1..140000."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        if len(out) % 3 == 2:
            cols = int(round(2 ** rng.uniform(15, np.log2(140000))))
            rows = int(round(2 ** rng.uniform(0, np.log2(max(1, max_elems // cols)))))
        else:
            rows = int(round(2 ** rng.uniform(0, np.log2(20000))))
            cols = int(round(2 ** rng.uniform(0, np.log2(140000))))
        if rows * cols <= max_elems:
            out.append((rows, cols))
    return out


@pytest.mark.parametrize("op", OPS)
def test_selected_plans_on_random_shapes_f32(gpu_device, op):
    import torch
    for i, (rows, cols) in enumerate(shapes(8000 + OPS.index(op), 6)):
        a = family_host_inputs(op, rows, cols, seed=9000 + i)
        ref = run_oracle(op, a)
        d = to_dev(a, gpu_device)
        key = plans.plan_key(rr.rr_select_plan(op, rows, cols))
        announce(f"fuzz {op} {rows}x{cols} {key}")
        compare(op, run_f32(op, d, None, None, gpu_device), ref, f"fuzz {op} {rows}x{cols} {key}")
        nbytes = rr.rr_workspace_bytes(op, rows, cols)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu_device)
            announce(f"fuzz {op} {rows}x{cols} with workspace")
            compare(op, run_f32(op, d, None, ws, gpu_device), ref, f"fuzz {op} {rows}x{cols} ws")


@pytest.mark.parametrize("op", OPS)
def test_selected_plans_on_random_shapes_bf16(gpu_device, op):
    import torch
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    for i, (rows, cols) in enumerate(shapes(8100 + OPS.index(op), 6)):
        if i % 2:
            cols = max(8, cols - cols % 8)      # half the draws allow 8-wide packs
        d = workloads.family_inputs_bf16(rows, cols, seed=9100 + i)
        ref = run_oracle_bf16(op, d, eps)
        t = dev_inputs_bf16(d, gpu_device)
        key = plans.plan_key(rr.rr_select_plan(op + "_bf16", rows, cols))
        announce(f"fuzz {op}_bf16 {rows}x{cols} {key}")
        compare_bf16(rename(run_bf16(op, t, None, None)), ref, f"fuzz {op}_bf16 {rows}x{cols} {key}")
        nbytes = rr.rr_workspace_bytes(op + "_bf16", rows, cols)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu_device)
            announce(f"fuzz {op}_bf16 {rows}x{cols} with workspace")
            compare_bf16(rename(run_bf16(op, t, None, ws)), ref, f"fuzz {op}_bf16 {rows}x{cols} ws")


@pytest.mark.parametrize("op", OPS)
def test_random_legal_plans_on_random_shapes(gpu_device, op):
    """Two random legal plans of the candidate grid (every path, pack width,
    slot count and cache policy the grid holds) per random shape, float and
    bfloat16 storage."""
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    rng = np.random.default_rng(8200 + OPS.index(op))
    for i, (rows, cols) in enumerate(shapes(8300 + OPS.index(op), 4, max_elems=1 << 21)):
        a = family_host_inputs(op, rows, cols, seed=9200 + i)
        ref = run_oracle(op, a)
        d = to_dev(a, gpu_device)
        cands = plans.candidate_plans(op, rows, cols, caches=(0, 1, 2))
        for j in rng.choice(len(cands), size=min(2, len(cands)), replace=False):
            p = cands[int(j)]
            what = f"fuzz-plan {op} {rows}x{cols} {plans.plan_key(p)}"
            announce(what)
            compare(op, run_f32(op, d, p, None, gpu_device), ref, what)
        cols8 = max(8, cols - cols % 8)
        db = workloads.family_inputs_bf16(rows, cols8, seed=9300 + i)
        refb = run_oracle_bf16(op, db, eps)
        t = dev_inputs_bf16(db, gpu_device)
        cands = plans.candidate_plans(op + "_bf16", rows, cols8, caches=(0, 1, 2))
        for j in rng.choice(len(cands), size=min(2, len(cands)), replace=False):
            p = cands[int(j)]
            what = f"fuzz-plan {op}_bf16 {rows}x{cols8} {plans.plan_key(p)}"
            announce(what)
            compare_bf16(rename(run_bf16(op, t, p, None)), refb, what)


@pytest.mark.parametrize("op", ["softmax", "cross_entropy"])
def test_masked_rows_on_random_shapes(gpu_device, op):
    """Random shapes with a random fraction (0 to 95 %) of -inf entries per
    row, some rows masked in one contiguous run and one row fully masked,
    with the selected plan and, where the selector splits, with a
    workspace; cross-entropy targets point at unmasked entries except in
    the fully masked row."""
    import torch
    rng = np.random.default_rng(8400 + (op == "softmax"))
    for i, (rows, cols) in enumerate(shapes(8500 + (op == "softmax"), 6)):
        a = family_host_inputs(op, rows, cols, seed=9400 + i)
        x = a["x"]
        for r in range(rows):
            if r % 3 == 1 and cols > 2:
                lo = int(rng.integers(0, cols - 1))
                x[r, lo:int(rng.integers(lo + 1, cols))] = -np.inf
            else:
                x[r, rng.random(cols) < rng.uniform(0, 0.95)] = -np.inf
        full = int(rng.integers(0, rows))
        x[full, :] = -np.inf
        if op == "cross_entropy":
            t = a["targets"]
            for r in range(rows):
                alive = np.flatnonzero(np.isfinite(x[r]))
                t[r] = int(rng.choice(alive)) if alive.size else 0
        ref = run_oracle(op, a)
        d = to_dev(a, gpu_device)
        key = plans.plan_key(rr.rr_select_plan(op, rows, cols))
        what = f"fuzz-masked {op} {rows}x{cols} {key}"
        announce(what)
        compare(op, run_f32(op, d, None, None, gpu_device), ref, what)
        nbytes = rr.rr_workspace_bytes(op, rows, cols)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu_device)
            announce(what + " with workspace")
            compare(op, run_f32(op, d, None, ws, gpu_device), ref, what + " ws")


def test_long_campaign(gpu_device):
    """Opt-in, time-bounded campaign (ROWRED_FUZZ_SECONDS; ROWRED_FUZZ_SEED
    picks the seeds): round after round of random shapes for every operator,
    each checked against the oracle with the selected plan (with and without
    a workspace), three random legal plans of the candidate grid, random
    explicit split plans, for the per-element operators one random plan
    with y aliasing x (split plans included) and, for RMSNorm, the
    allocation-free entry point; bfloat16 storage with the selected plan,
    three random plans and one in place. Every mismatch is collected and
    reported together."""
    import torch
    budget = float(os.environ.get("ROWRED_FUZZ_SECONDS", "0"))
    if budget <= 0:
        pytest.skip("set ROWRED_FUZZ_SECONDS to run the long campaign")
    base = int(os.environ.get("ROWRED_FUZZ_SEED", "50000"))
    t0 = time.time()
    fails, n = [], 0

    def check(what, fn):
        nonlocal n
        n += 1
        try:
            fn()
        except AssertionError as e:
            fails.append(f"{what}: {str(e)[:300]}")

    rnd = 0
    while time.time() - t0 < budget:
        for k, op in enumerate(OPS):
            eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
            rng = np.random.default_rng(base + 97 * rnd + k)
            for i, (rows, cols) in enumerate(shapes(base + 1000 * rnd + 10 * k, 4, max_elems=1 << 21)):
                seed = base + 100000 * rnd + 1000 * k + i
                a = family_host_inputs(op, rows, cols, seed=seed)
                ref = run_oracle(op, a)
                d = to_dev(a, gpu_device)
                check(f"selected {op} {rows}x{cols}",
                      lambda: compare(op, run_f32(op, d, None, None, gpu_device), ref, "selected"))
                nb = rr.rr_workspace_bytes(op, rows, cols)
                if nb > 0:
                    ws = torch.empty(nb, dtype=torch.uint8, device=gpu_device)
                    check(f"workspace {op} {rows}x{cols}",
                          lambda: compare(op, run_f32(op, d, None, ws, gpu_device), ref, "workspace"))
                cands = plans.candidate_plans(op, rows, cols, caches=(0, 1, 2))
                for j in rng.choice(len(cands), size=min(3, len(cands)), replace=False):
                    p = cands[int(j)]
                    check(f"plan {op} {rows}x{cols} {plans.plan_key(p)}",
                          lambda: compare(op, run_f32(op, d, p, None, gpu_device), ref, "plan"))
                for lanes, slots in ((64, 16), (128, 32), (256, 16), (512, 32), (1024, 16), (1024, 32)):
                    sp = rr.rr_plan(3, lanes, lanes, 1, 4, slots, 2)
                    if rr.rr_check_plan(op, rows, cols, sp) == 0 and rng.random() < 0.5:
                        ws = torch.empty(rr.rr_workspace_bytes(op, rows, cols, sp), dtype=torch.uint8,
                                         device=gpu_device)
                        check(f"split {op} {rows}x{cols} {plans.plan_key(sp)}",
                              lambda: compare(op, run_f32(op, d, sp, ws, gpu_device), ref, "split"))
                if op in IN_PLACE_OPS:
                    splits = [rr.rr_plan(3, w, w, 1, 4, k, 2) for w in (64, 256, 1024) for k in (16, 32)]
                    pool = cands + [sp for sp in splits if rr.rr_check_plan(op, rows, cols, sp) == 0]
                    p = pool[int(rng.integers(0, len(pool)))]
                    ws = None
                    if p.path == 3:
                        ws = torch.empty(rr.rr_workspace_bytes(op, rows, cols, p), dtype=torch.uint8,
                                         device=gpu_device)
                    fresh = to_dev(a, gpu_device)
                    check(f"in-place {op} {rows}x{cols} {plans.plan_key(p)}",
                          lambda: compare(op, run_in_place(op, fresh, p, ws, False), ref, "in-place"))
                if op == "rmsnorm":
                    y = torch.empty_like(d["x"])

                    def no_alloc():
                        got = rr.rmsnorm_f32_noalloc(d["x"], d["w"], float(a["eps"]), y)
                        torch.cuda.synchronize()
                        compare(op, {"y": got}, ref, "no-alloc")
                    check(f"no-alloc {rows}x{cols}", no_alloc)
                c8 = max(8, cols - cols % 8) if i % 2 else cols
                db = workloads.family_inputs_bf16(rows, c8, seed=seed + 7)
                refb = run_oracle_bf16(op, db, eps)
                t = dev_inputs_bf16(db, gpu_device)
                name = op + "_bf16"
                check(f"selected {name} {rows}x{c8}",
                      lambda: compare_bf16(rename(run_bf16(op, t, None, None)), refb, "selected"))
                cands = plans.candidate_plans(name, rows, c8, caches=(0, 1, 2))
                for j in rng.choice(len(cands), size=min(3, len(cands)), replace=False):
                    p = cands[int(j)]
                    check(f"plan {name} {rows}x{c8} {plans.plan_key(p)}",
                          lambda: compare_bf16(rename(run_bf16(op, t, p, None)), refb, "plan"))
                if op in IN_PLACE_OPS:
                    splits = [rr.rr_plan(3, w, w, 1, 8, k, 2) for w in (64, 256, 1024) for k in (16, 32)]
                    pool = cands + [sp for sp in splits if rr.rr_check_plan(name, rows, c8, sp) == 0]
                    p = pool[int(rng.integers(0, len(pool)))]
                    ws = None
                    if p.path == 3:
                        ws = torch.empty(rr.rr_workspace_bytes(name, rows, c8, p), dtype=torch.uint8,
                                         device=gpu_device)
                    fresh = dict(dev_inputs_bf16(db, gpu_device), eps=eps)
                    fresh["w"] = fresh["gamma"]
                    check(f"in-place {name} {rows}x{c8} {plans.plan_key(p)}",
                          lambda: compare_bf16(rename(run_in_place(op, fresh, p, ws, True)), refb, "in-place"))
            announce(f"long campaign: round {rnd} {op}, {n} checks, {len(fails)} mismatches, "
                     f"{time.time() - t0:.0f} s")
        rnd += 1
    assert not fails, f"{len(fails)} of {n} checks failed:\n" + "\n".join(fails[:20])

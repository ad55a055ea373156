"""GPU parity of the split-row path (several workgroups per row, partials in
a caller workspace, two launches) against the CPU oracle, for every operator
in float and bfloat16 storage, with the selector's split plans and explicit
ones, ragged last slices, determinism, and workspace reuse."""
import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import workloads
from row_reduction_amd._capi import RR_PATH_SPLIT

from parity_util import announce, compare, family_host_inputs, run_oracle
from test_gpu_bf16 import compare as compare_bf16
from test_gpu_bf16 import dev_inputs as dev_inputs_bf16
from test_gpu_bf16 import run_oracle as run_oracle_bf16

pytestmark = pytest.mark.gpu

OPS = list(workloads.OPS)
SPLIT_SHAPES = [(1, 100003), (3, 40000), (17, 16384), (2, 1 << 20)]
SPLIT_SHAPES_BF16 = [(1, 100000), (3, 40000), (17, 16384), (2, 1 << 20)]


def split_plans(op, rows, cols):
    """Explicit split plans legal for the shape."""
    v = 8 if op.endswith("_bf16") else 4
    out = []
    for lanes, slots in [(64, 16), (128, 16), (256, 16), (512, 16), (256, 32), (1024, 32)]:
        p = rr.rr_plan(RR_PATH_SPLIT, lanes, lanes, 1, v, slots, 2)
        if rr.rr_check_plan(op, rows, cols, p) == 0:
            out.append(p)
    return out


def run_f32(op, d, plan, ws, gpu_device):
    import torch
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(gpu_device) if isinstance(v, np.ndarray) else v
         for k, v in d.items()}
    if op == "rmsnorm":
        return {"y": rr.rmsnorm_f32(t["x"], t["w"], t["eps"], plan=plan, workspace=ws)}
    if op == "sum":
        return {"out": rr.row_sum_f32(t["x"], plan=plan, workspace=ws)}
    if op == "softmax":
        return {"y": rr.softmax_f32(t["x"], plan=plan, workspace=ws)}
    if op == "layernorm":
        return {"y": rr.layernorm_f32(t["x"], t["w"], t["beta"], t["eps"], plan=plan, workspace=ws)}
    if op == "residual_layernorm":
        h = torch.empty_like(t["x"])
        y = rr.residual_layernorm_f32(t["x"], t["residual"], t["w"], t["beta"], t["eps"], h_out=h,
                                      plan=plan, workspace=ws)
        return {"y": y, "h": h}
    return {"loss": rr.cross_entropy_f32(t["x"], t["targets"], plan=plan, workspace=ws)}


def run_bf16(op, t, plan, ws):
    import torch
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    if op == "rmsnorm":
        return {"y": rr.rmsnorm_bf16(t["x"], t["gamma"], eps, plan=plan, workspace=ws)}
    if op == "sum":
        return {"out": rr.row_sum_bf16(t["x"], plan=plan, workspace=ws)}
    if op == "softmax":
        return {"y": rr.softmax_bf16(t["x"], plan=plan, workspace=ws)}
    if op == "layernorm":
        return {"y": rr.layernorm_bf16(t["x"], t["gamma"], t["beta"], eps, plan=plan, workspace=ws)}
    if op == "residual_layernorm":
        h = torch.empty_like(t["x"])
        y = rr.residual_layernorm_bf16(t["x"], t["residual"], t["gamma"], t["beta"], eps, h_out=h,
                                       plan=plan, workspace=ws)
        return {"y": y, "h": h}
    return {"loss": rr.cross_entropy_bf16(t["x"], t["targets"], plan=plan, workspace=ws)}


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_split_f32_matches_oracle(gpu_device, op, shape):
    import torch
    rows, cols = shape
    d = family_host_inputs(op, rows, cols, seed=cols % 997)
    ref = run_oracle(op, d)
    sel = rr.rr_select_plan(op, rows, cols)
    # With a workspace the selector splits where its cost model predicts the
    # split faster (the plain plan otherwise); explicit split plans follow.
    nbytes = rr.rr_workspace_bytes(op, rows, cols)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=gpu_device)
    announce(f"split {op} {rows}x{cols} auto (workspace {nbytes} B; plain plan {sel.as_dict()})")
    compare(op, run_f32(op, d, None, ws, gpu_device), ref, f"split {op} {rows}x{cols} auto")
    for p in split_plans(op, rows, cols):
        need = rr.rr_workspace_bytes(op, rows, cols, p)
        wsp = torch.empty(need, dtype=torch.uint8, device=gpu_device)
        what = f"split {op} {rows}x{cols} w{p.lanes_per_row} k{p.slots}"
        announce(what)
        compare(op, run_f32(op, d, p, wsp, gpu_device), ref, what)


@pytest.mark.parametrize("shape", SPLIT_SHAPES_BF16)
@pytest.mark.parametrize("op", OPS)
def test_split_bf16_matches_oracle(gpu_device, op, shape):
    import torch
    rows, cols = shape
    d = workloads.family_inputs_bf16(rows, cols, seed=cols % 991)
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    ref = run_oracle_bf16(op, d, eps)
    t = dev_inputs_bf16(d, gpu_device)
    nbytes = rr.rr_workspace_bytes(op + "_bf16", rows, cols)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=gpu_device)
    announce(f"split {op}_bf16 {rows}x{cols} auto")
    compare_bf16(run_bf16(op, t, None, ws), ref, f"split {op}_bf16 {rows}x{cols} auto")
    for p in split_plans(op + "_bf16", rows, cols):
        need = rr.rr_workspace_bytes(op + "_bf16", rows, cols, p)
        wsp = torch.empty(need, dtype=torch.uint8, device=gpu_device)
        what = f"split {op}_bf16 {rows}x{cols} w{p.lanes_per_row} k{p.slots}"
        announce(what)
        compare_bf16(run_bf16(op, t, p, wsp), ref, what)


def test_split_deterministic_and_workspace_reuse(gpu_device):
    """Fixed merge order: repeated split calls are bit-identical, and one
    workspace serves calls of different shapes in sequence."""
    import torch
    ws = torch.empty(rr.rr_workspace_bytes("softmax", 4, 1 << 20), dtype=torch.uint8, device=gpu_device)
    for op in OPS:
        d = family_host_inputs(op, 4, 1 << 20, seed=5)
        announce(f"split determinism {op}")
        first = {k: v.clone() for k, v in run_f32(op, d, None, ws, gpu_device).items()}
        for _ in range(5):
            again = run_f32(op, d, None, ws, gpu_device)
            for k in first:
                assert torch.equal(first[k].view(torch.int32), again[k].view(torch.int32)), op
    d = family_host_inputs("rmsnorm", 2, 50000, seed=6)
    compare("rmsnorm", run_f32("rmsnorm", d, None, ws, gpu_device), run_oracle("rmsnorm", d),
            "split rmsnorm 2x50000 reused workspace")


IN_PLACE_OPS = ["rmsnorm", "softmax", "layernorm", "residual_layernorm"]


def run_in_place(op, t, plan, ws, bf16):
    """One call with y aliasing x (residual LayerNorm: h_out in its own buffer)."""
    import torch
    eps = t.get("eps")
    x = t["x"]
    sfx = "_bf16" if bf16 else "_f32"
    if op == "rmsnorm":
        getattr(rr, "rmsnorm" + sfx)(x, t["w"], eps, y=x, plan=plan, workspace=ws)
        return {"y": x}
    if op == "softmax":
        getattr(rr, "softmax" + sfx)(x, y=x, plan=plan, workspace=ws)
        return {"y": x}
    if op == "layernorm":
        getattr(rr, "layernorm" + sfx)(x, t["w"], t["beta"], eps, y=x, plan=plan, workspace=ws)
        return {"y": x}
    h = torch.empty_like(x)
    getattr(rr, "residual_layernorm" + sfx)(x, t["residual"], t["w"], t["beta"], eps, y=x, h_out=h,
                                           plan=plan, workspace=ws)
    return {"y": x, "h": h}


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("op", IN_PLACE_OPS)
def test_split_in_place(gpu_device, op, bf16):
    """y aliasing x is safe on split rows for every per-element operator: the
    second launch's workgroups read only their own slice's columns (the
    LayerNorms' shift is each slice's own first value, taken in the first
    launch, which writes no input), for every explicit split plan and the
    selected one, with slices that finish at different times (many rows,
    narrow slices)."""
    import torch
    rows, cols = 5, 100000
    name = op + ("_bf16" if bf16 else "")
    if bf16:
        d = workloads.family_inputs_bf16(rows, cols, seed=11)
        eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
        ref = run_oracle_bf16(op, d, eps)
        fresh = lambda: dict(dev_inputs_bf16(d, gpu_device), w=None, eps=eps)
    else:
        d = family_host_inputs(op, rows, cols, seed=11)
        ref = run_oracle(op, d)
        fresh = lambda: {k: (torch.from_numpy(np.ascontiguousarray(v)).to(gpu_device)
                             if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    plans = [None] + split_plans(name, rows, cols)
    assert len(plans) >= 4
    for p in plans:
        t = fresh()
        if bf16:
            t["w"] = t["gamma"]
        need = rr.rr_workspace_bytes(name, rows, cols, p)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=gpu_device)
        what = f"split {name} {rows}x{cols} in place " + (f"w{p.lanes_per_row} k{p.slots}" if p else "selected")
        announce(what)
        got = run_in_place(op, t, p, ws, bf16)
        if bf16:
            compare_bf16(got, ref, what)
        else:
            compare(op, got, ref, what)

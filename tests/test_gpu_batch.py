"""GPU parity of the batched launch (rr_batch): several problems of any
operators, shapes and storage types in one kernel launch, every output
compared element by element with the CPU oracle at the operators' own
tolerances; zero-row problems, the size limit, both pack widths, and HIP-graph
replay of a batch."""
import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import workloads

from parity_util import announce, compare, family_host_inputs, run_oracle, to_dev
from test_gpu_bf16 import compare as compare_bf16
from test_gpu_bf16 import dev_inputs as dev_inputs_bf16
from test_gpu_bf16 import run_oracle as run_oracle_bf16

pytestmark = pytest.mark.gpu

OPS = list(workloads.OPS)


def f32_problem(op, d):
    kw = {}
    if op in ("rmsnorm", "layernorm", "residual_layernorm"):
        kw.update(w=d["w"], eps=d["eps"])
    if op in ("layernorm", "residual_layernorm"):
        kw["beta"] = d["beta"]
    if op == "residual_layernorm":
        import torch
        kw.update(residual=d["residual"], h_out=torch.empty_like(d["x"]))
    if op == "cross_entropy":
        kw["targets"] = d["targets"]
    return rr.batch_problem(op, d["x"], **kw)


def bf16_problem(op, t):
    kw = {}
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    if op in ("rmsnorm", "layernorm", "residual_layernorm"):
        kw.update(w=t["gamma"], eps=eps)
    if op in ("layernorm", "residual_layernorm"):
        kw["beta"] = t["beta"]
    if op == "residual_layernorm":
        import torch
        kw.update(residual=t["residual"], h_out=torch.empty_like(t["x"]))
    if op == "cross_entropy":
        kw["targets"] = t["targets"]
    return rr.batch_problem(op + "_bf16", t["x"], **kw)


def rename(outs):
    """batch_problem's output names to the parity helpers' names."""
    got = dict(outs)
    if "out" in got:
        got["loss"] = got["out"]
    return got


def run_f32_batch(specs, device, what):
    """specs: [(op, rows, cols, seed)]; returns nothing, asserts parity."""
    items, probs = [], []
    for op, rows, cols, seed in specs:
        a = family_host_inputs(op, rows, cols, seed)
        d = to_dev(a, device)          # kept in `items`: the batch reads it later
        p, outs = f32_problem(op, d)
        items.append((op, rows, cols, a, outs, d))
        probs.append(p)
    announce(f"{what}: rr_batch of {len(probs)} problems")
    rr.rr_batch(probs)
    for op, rows, cols, a, outs, _ in items:
        if rows == 0:
            continue
        ref = run_oracle(op, a)
        if op == "sum":
            ref = {"out": ref["out"]}
        compare(op, rename(outs), ref, f"{what} {op} {rows}x{cols}")
    return items


def test_pages_operator_coverage_in_one_launch(gpu_device):
    """The pages' operator-coverage set (five operators on four shapes) plus
    RMSNorm on the same shapes: 24 problems, one launch."""
    specs = [(op, r, c, 100 + i) for i, (r, c) in enumerate(workloads.FAMILY_SHAPES) for op in OPS]
    assert len(specs) == 24
    run_f32_batch(specs, gpu_device, "coverage")


@pytest.mark.parametrize("cols", [1, 2, 3, 4, 5, 7, 8, 31, 33, 127, 128, 129, 257, 4103])
def test_ragged_widths_both_pack_widths(gpu_device, cols):
    specs = [(op, r, cols, 7 * cols + i) for i, (op, r) in enumerate(zip(OPS, (1, 3, 5, 2, 4, 6)))]
    run_f32_batch(specs, gpu_device, f"ragged {cols}")


def test_bf16_and_float_mixed(gpu_device):
    import torch
    probs, checks = [], []
    for i, (op, rows, cols) in enumerate([("rmsnorm", 17, 257), ("softmax", 5, 4096), ("layernorm", 3, 1000),
                                         ("residual_layernorm", 9, 264), ("sum", 4, 4103),
                                         ("cross_entropy", 6, 129)]):
        d = workloads.family_inputs_bf16(rows, cols, seed=300 + i)
        eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
        t = dev_inputs_bf16(d, gpu_device)
        p, outs = bf16_problem(op, t)
        probs.append(p)
        checks.append(("bf16", op, rows, cols, run_oracle_bf16(op, d, eps), outs, t))
        a = family_host_inputs(op, rows + 1, cols + 3, 400 + i)
        dev = to_dev(a, gpu_device)
        p, outs = f32_problem(op, dev)
        probs.append(p)
        checks.append(("f32", op, rows + 1, cols + 3, run_oracle(op, a), outs, dev))
    announce(f"mixed bf16/f32 rr_batch of {len(probs)} problems")
    rr.rr_batch(probs)
    for kind, op, rows, cols, ref, outs, _ in checks:
        what = f"mixed {kind} {op} {rows}x{cols}"
        if kind == "bf16":
            compare_bf16(rename(outs), ref, what)
        else:
            compare(op, rename(outs), ref, what)
    torch.cuda.synchronize()


def test_zero_row_problems_and_full_batch(gpu_device):
    specs = []
    for i in range(rr._capi.RR_BATCH_MAX):
        op = OPS[i % len(OPS)]
        rows = 0 if i % 7 == 3 else 1 + (i % 5)
        specs.append((op, rows, 33 + 17 * i, 500 + i))
    run_f32_batch(specs, gpu_device, "full batch")


def test_batch_equals_eager_under_graph_replay(gpu_device):
    """A captured batch replays to the same outputs as the eager batch."""
    import torch
    specs = [(op, r, c, 600 + i) for i, (r, c) in enumerate([(17, 257), (64, 4096)]) for op in OPS]
    items, probs = [], []
    for op, rows, cols, seed in specs:
        d = to_dev(family_host_inputs(op, rows, cols, seed), gpu_device)
        p, outs = f32_problem(op, d)
        items.append((d, outs))
        probs.append(p)
    announce("batch eager")
    rr.rr_batch(probs)
    torch.cuda.synchronize()
    eager = [{k: v.clone() for k, v in outs.items()} for _, outs in items]
    for _, outs in items:
        for v in outs.values():
            v.zero_()
    announce("batch graph capture")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rr.rr_batch(probs)           # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        rr.rr_batch(probs)
    for rep in range(3):
        for _, outs in items:
            for v in outs.values():
                v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, (_, outs) in zip(eager, items):
            for k in e:
                assert torch.equal(e[k], outs[k]), (rep, k)

"""LayerNorm and residual LayerNorm on ill-conditioned rows — variance tiny
next to mean^2, very short rows of nearly equal values, a first value far
from the mean — on every path (register, streaming with and without kept
slots, split rows, the batched launch) in both storage types, compared with
the float64 oracle at the operators' usual tolerances. A float32 row mean
would miss these by its own rounding error (about 2^-24 |mean|) divided by
sqrt(var + eps)."""
import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import plans, workloads

from parity_util import announce, assert_close
from test_gpu_bf16 import assert_bf16_close, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

EPS = workloads.LAYERNORM_EPS


def rows_of(kind, rows, cols, seed):
    rng = np.random.default_rng(seed)
    if kind == "near_equal":          # short rows of nearly equal values around a large offset
        base = rng.uniform(-50, 50, (rows, 1))
        x = base + rng.normal(0, 1e-3, (rows, cols))
    elif kind == "big_mean":          # mean 1000, spread 0.01
        x = 1000.0 + rng.normal(0, 1e-2, (rows, cols))
    else:                             # "outlier_first": the first value 100 sigma out
        x = rng.normal(3.0, 0.5, (rows, cols))
        x[:, 0] += 50.0
    x = x.astype(np.float32)
    r = (rng.normal(0, 1e-3, (rows, cols))).astype(np.float32)
    g = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    b = rng.normal(0, 0.1, cols).astype(np.float32)
    return x, r, g, b


CASES = [("near_equal", 597, 2), ("near_equal", 301, 3), ("near_equal", 40, 8), ("big_mean", 5, 4096),
         ("big_mean", 3, 5000), ("big_mean", 2, 65536), ("big_mean", 2, 100003), ("outlier_first", 3, 4103),
         ("outlier_first", 2, 70001)]


def explicit_plans(op, rows, cols):
    out = [None]
    for p in plans.candidate_plans(op, rows, cols, include_loop=True):
        if p.path == 2 or p.lanes_per_row in (8, 64, 1024):
            out.append(p)
    return out[:12]


@pytest.mark.parametrize("kind,rows,cols", CASES)
@pytest.mark.parametrize("residual", [False, True])
def test_float_layernorm_ill_conditioned(gpu_device, kind, rows, cols, residual):
    import torch
    x, r, g, b = rows_of(kind, rows, cols, seed=cols + rows)
    if residual:
        ref, href = oracle.residual_layernorm(x, r, g, b, EPS)
    else:
        ref = oracle.layernorm(x, g, b, EPS)
    dx, dr, dg, db = (torch.from_numpy(a).to(gpu_device) for a in (x, r, g, b))
    op = "residual_layernorm" if residual else "layernorm"
    for p in explicit_plans(op, rows, cols):
        what = f"{op} {kind} {rows}x{cols} {plans.plan_key(p) if p else 'selected'}"
        announce(what)
        if residual:
            y = rr.residual_layernorm_f32(dx, dr, dg, db, EPS, plan=p)
        else:
            y = rr.layernorm_f32(dx, dg, db, EPS, plan=p)
        assert_close(y.cpu().numpy(), ref, what)
    ws = rr.workspace_for(op, rows, cols, device=gpu_device)
    if ws is not None:
        announce(f"{op} {kind} {rows}x{cols} split")
        y = (rr.residual_layernorm_f32(dx, dr, dg, db, EPS, workspace=ws) if residual
             else rr.layernorm_f32(dx, dg, db, EPS, workspace=ws))
        assert_close(y.cpu().numpy(), ref, f"{op} {kind} {rows}x{cols} split")
    kw = dict(w=dg, beta=db, eps=EPS)
    if residual:
        kw["residual"] = dr
    prob, outs = rr.batch_problem(op, dx, **kw)
    announce(f"{op} {kind} {rows}x{cols} batch")
    rr.rr_batch([prob])
    assert_close(outs["y"].cpu().numpy(), ref, f"{op} {kind} {rows}x{cols} batch")


@pytest.mark.parametrize("kind,rows,cols", [c for c in CASES if c[2] % 8 == 0 or c[2] < 9])
def test_bf16_layernorm_ill_conditioned(gpu_device, kind, rows, cols):
    import torch
    x, r, g, b = rows_of(kind, rows, cols, seed=7 * cols + rows)
    xb, gb, bb = (workloads.as_bf16_bits(a) for a in (x, g, b))
    ref = oracle.layernorm_bf16(xb, gb, bb, EPS)
    dx, dg, db = (to_dev_bf16(a, gpu_device) for a in (xb, gb, bb))
    for p in explicit_plans("layernorm_bf16", rows, cols):
        what = f"layernorm_bf16 {kind} {rows}x{cols} {plans.plan_key(p) if p else 'selected'}"
        announce(what)
        y = rr.layernorm_bf16(dx, dg, db, EPS, plan=p)
        assert_bf16_close(from_dev_bf16(y), ref, what)
    ws = rr.workspace_for("layernorm_bf16", rows, cols, device=gpu_device)
    if ws is not None:
        announce(f"layernorm_bf16 {kind} {rows}x{cols} split")
        y = rr.layernorm_bf16(dx, dg, db, EPS, workspace=ws)
        assert_bf16_close(from_dev_bf16(y), ref, f"layernorm_bf16 {kind} {rows}x{cols} split")

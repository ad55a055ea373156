"""GPU parity: every output element of the HIP path against the CPU oracle,
within |err| <= 1e-5 + 1e-5 |ref| (bit-exact where the arithmetic is exact).

Covers the five measured configurations at their full sizes with the plans
the library selects (the launch configuration the benchmark times), every
legal plan of the search grid on the ragged test matrix the LuisaCompute
"Consecutive-worker reduction layout checkpoint" page lists in its
"Verification checkpoint" section (N = 1, 31, 33, 127, 128, 129, 257, 4103;
packed short rows and multi-wavefront rows), the streaming path beyond the
register budget, and the special cases of each operator.
"""
import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import plans, workloads

from parity_util import (announce, assert_close, compare, family_host_inputs, host_inputs,
                         run_gpu, run_oracle, to_dev)

pytestmark = pytest.mark.gpu

OPS = list(workloads.OPS)
MATRIX_N = (1, 31, 33, 127, 128, 129, 257, 4103)


# ---------------------------------------------------------------- measured configurations

@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_rmsnorm_configs_full_size(gpu_device, k):
    for wl in workloads.config_workloads(k):
        announce(f"rmsnorm config {k} {wl.rows}x{wl.cols} plan={rr.rr_select_plan('rmsnorm', wl.rows, wl.cols)}")
        a = host_inputs("rmsnorm", wl.x, w=wl.w, eps=wl.eps)
        got = run_gpu("rmsnorm", to_dev(a, gpu_device))
        compare("rmsnorm", got, run_oracle("rmsnorm", a), f"rmsnorm {wl.name}")


@pytest.mark.parametrize("shape", workloads.FAMILY_SHAPES)
@pytest.mark.parametrize("op", [o for o in OPS if o != "rmsnorm"])
def test_family_config_full_size(gpu_device, op, shape):
    rows, cols = shape
    announce(f"family {op} {rows}x{cols} plan={rr.rr_select_plan(op, rows, cols)}")
    a = family_host_inputs(op, rows, cols, seed=1005)
    got = run_gpu(op, to_dev(a, gpu_device), with_h=True)
    compare(op, got, run_oracle(op, a), f"{op} {rows}x{cols}")


# ---------------------------------------------------------------- every plan, ragged matrix

@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("cols", MATRIX_N)
def test_every_legal_plan_on_ragged_matrix(gpu_device, op, cols):
    for rows in (1, 5):
        a = family_host_inputs(op, rows, cols, seed=7 + cols)
        ref = run_oracle(op, a)
        d = to_dev(a, gpu_device)
        for p in plans.candidate_plans(op, rows, cols):
            what = f"{op} {rows}x{cols} {plans.plan_key(p)}"
            announce(what)
            got = run_gpu(op, d, plan=p, with_h=True)
            compare(op, got, ref, what)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("cols", [129, 4096, 33000])
def test_cache_policies_give_identical_results(gpu_device, op, cols):
    """Non-temporal hints change where data is cached, never the arithmetic:
    every cache policy of a plan must reproduce the default bit for bit."""
    import torch
    rows = 5
    a = family_host_inputs(op, rows, cols, seed=31)
    ref = run_oracle(op, a)
    d = to_dev(a, gpu_device)
    base = [p for p in plans.candidate_plans(op, rows, cols) if p.v == 4 or p.path == 2]
    for p in base[::3]:
        outs = []
        for cache in (0, 1, 2):
            q = rr.rr_plan.from_dict({**p.as_dict(), "cache": cache})
            what = f"{op} {rows}x{cols} {plans.plan_key(q)}"
            announce(what)
            got = run_gpu(op, d, plan=q, with_h=True)
            compare(op, got, ref, what)
            outs.append({k: v.clone() for k, v in got.items()})
        for o in outs[1:]:
            for k in o:
                assert torch.equal(o[k].view(torch.int32), outs[0][k].view(torch.int32)), (op, k)


@pytest.mark.parametrize("op", OPS)
def test_many_packed_rows_and_partial_last_group(gpu_device, op):
    rows, cols = 1003, 24          # 1003 rows: the last group is partly empty
    a = family_host_inputs(op, rows, cols, seed=5)
    ref = run_oracle(op, a)
    d = to_dev(a, gpu_device)
    for p in plans.candidate_plans(op, rows, cols, include_loop=False):
        what = f"{op} {rows}x{cols} {plans.plan_key(p)}"
        announce(what)
        compare(op, run_gpu(op, d, plan=p, with_h=True), ref, what)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("cols", [32768, 32769, 100003])
def test_streaming_path_beyond_register_budget(gpu_device, op, cols):
    rows = 3
    a = family_host_inputs(op, rows, cols, seed=9)
    ref = run_oracle(op, a)
    d = to_dev(a, gpu_device)
    p = rr.rr_select_plan(op, rows, cols)
    announce(f"{op} {rows}x{cols} selected {plans.plan_key(p)}")
    compare(op, run_gpu(op, d, with_h=True), ref, f"{op} {rows}x{cols} selected")
    for v in (1, 2, 4):
        for block in (256, 1024):
            for kept in (0, 32, 64, 96):
                lp = rr.rr_plan(2, block, block, 1, v, kept)
                if rr.rr_check_plan(op, rows, cols, lp) != 0:
                    continue
                what = f"{op} {rows}x{cols} {plans.plan_key(lp)}"
                announce(what)
                compare(op, run_gpu(op, d, plan=lp, with_h=True), ref, what)


@pytest.mark.parametrize("op", ["rmsnorm", "softmax", "layernorm", "residual_layernorm"])
@pytest.mark.parametrize("cols", [4, 129, 1000, 4096, 5000, 8191])
def test_streaming_kept_slots_on_short_rows(gpu_device, op, cols):
    """Kept register chunks beyond the row's last chunk (fewer chunks than the
    plan keeps) read in bounds, count nothing and store nothing."""
    rows = 5
    a = family_host_inputs(op, rows, cols, seed=19)
    ref = run_oracle(op, a)
    d = to_dev(a, gpu_device)
    for block, kept in ((256, 32), (1024, 32), (1024, 64), (1024, 96)):
        lp = rr.rr_plan(2, block, block, 1, 4, kept)
        if rr.rr_check_plan(op, rows, cols, lp) != 0:
            continue
        what = f"{op} {rows}x{cols} {plans.plan_key(lp)}"
        announce(what)
        compare(op, run_gpu(op, d, plan=lp, with_h=True), ref, what)


# ---------------------------------------------------------------- semantics and special cases

def test_rmsnorm_in_place(gpu_device):
    import torch
    wl = workloads.rmsnorm_workload(64, 4096, seed=21)
    ref = oracle.rmsnorm(wl.x, wl.w, wl.eps)
    x = torch.from_numpy(wl.x).to(gpu_device)
    w = torch.from_numpy(wl.w).to(gpu_device)
    announce("rmsnorm in place 64x4096")
    rr.rmsnorm_f32(x, w, wl.eps, y=x)
    assert_close(x.cpu().numpy(), ref, "rmsnorm in place")


def test_softmax_in_place_ragged(gpu_device):
    import torch
    d = workloads.family_inputs(17, 257, seed=22)
    ref = oracle.softmax(d["x"])
    x = torch.from_numpy(d["x"]).to(gpu_device)
    announce("softmax in place 17x257")
    rr.softmax_f32(x, y=x)
    assert_close(x.cpu().numpy(), ref, "softmax in place")


def test_rmsnorm_unit_magnitude_bitwise(gpu_device):
    """x in {-1,+1}, w = 1, eps = 0: mean square is exactly 1, y = x bit for bit."""
    import torch
    rng = np.random.default_rng(3)
    for rows, cols in [(5, 257), (64, 4096), (3, 40000)]:
        x = np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0).astype(np.float32)
        xd = torch.from_numpy(x).to(gpu_device)
        wd = torch.ones(cols, dtype=torch.float32, device=gpu_device)
        announce(f"rmsnorm +-1 {rows}x{cols}")
        y = rr.rmsnorm_f32(xd, wd, 0.0).cpu().numpy()
        assert np.array_equal(y, x)


def test_rmsnorm_signed_zero_and_zero_row(gpu_device):
    import torch
    x = np.zeros((2, 129), np.float32)
    x[0, 0] = -0.0
    x[0, 5] = 3.0
    x[1, :] = -0.0
    w = np.ones(129, np.float32)
    announce("rmsnorm signed zeros")
    y = rr.rmsnorm_f32(torch.from_numpy(x).to(gpu_device), torch.from_numpy(w).to(gpu_device),
                       1e-6).cpu().numpy()
    assert np.signbit(y[0, 0]) and not np.signbit(y[0, 1])
    assert np.all(np.signbit(y[1])) and np.all(y[1] == 0)


def test_rmsnorm_scale_invariance_eps0(gpu_device):
    import torch
    wl = workloads.rmsnorm_workload(17, 257, seed=23)
    w = torch.from_numpy(wl.w).to(gpu_device)
    announce("rmsnorm scale invariance")
    y1 = rr.rmsnorm_f32(torch.from_numpy(wl.x).to(gpu_device), w, 0.0).cpu().numpy()
    for alpha in (2.0 ** -7, 3.5, 1000.0):
        xs = (wl.x.astype(np.float64) * alpha).astype(np.float32)
        y2 = rr.rmsnorm_f32(torch.from_numpy(xs).to(gpu_device), w, 0.0).cpu().numpy()
        assert_close(y2, y1, f"scale {alpha}")


def test_row_sum_integer_rows_bitwise_every_plan(gpu_device):
    import torch
    rng = np.random.default_rng(4)
    for rows, cols in [(5, 257), (64, 4096), (5, 4103)]:
        x = rng.integers(-100, 100, size=(rows, cols)).astype(np.float32)
        exact = x.astype(np.int64).sum(axis=1).astype(np.float32)
        xd = torch.from_numpy(x).to(gpu_device)
        for p in plans.candidate_plans("sum", rows, cols):
            announce(f"row sum integers {rows}x{cols} {plans.plan_key(p)}")
            assert np.array_equal(rr.row_sum_f32(xd, plan=p).cpu().numpy(), exact)


def test_row_sum_cancellation(gpu_device):
    """Rows whose sum nearly cancels: float64 accumulation keeps the relative bound."""
    import torch
    rng = np.random.default_rng(5)
    x = rng.normal(0, 2, size=(256, 4096)).astype(np.float32)
    x[:, -1] = -x[:, :-1].astype(np.float64).sum(axis=1).astype(np.float32)
    announce("row sum cancellation 256x4096")
    got = rr.row_sum_f32(torch.from_numpy(x).to(gpu_device)).cpu().numpy()
    assert_close(got, oracle.row_sum(x), "row sum cancellation")


def test_softmax_rows_sum_to_one(gpu_device):
    import torch
    d = workloads.family_inputs(1024, 4096, seed=24)
    announce("softmax row sums 1024x4096")
    y = rr.softmax_f32(torch.from_numpy(d["x"]).to(gpu_device)).cpu().numpy().astype(np.float64)
    assert np.all(y >= 0) and np.all(y <= 1)
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-5


def test_softmax_constant_rows(gpu_device):
    import torch
    for cols in (1, 31, 257, 4096, 40000):
        x = np.full((3, cols), -1.25, np.float32)
        announce(f"softmax constant {cols}")
        y = rr.softmax_f32(torch.from_numpy(x).to(gpu_device)).cpu().numpy()
        assert_close(y, np.full_like(x, 1.0 / cols), f"softmax constant {cols}")


def test_cross_entropy_out_of_range_targets_give_nan(gpu_device):
    import torch
    d = workloads.family_inputs(6, 257, seed=25)
    t = np.array([-1, 257, 0, 256, 1 << 30, 5], np.int32)
    announce("cross entropy bad targets")
    for p in [None] + plans.candidate_plans("cross_entropy", 6, 257)[:6]:
        loss = rr.cross_entropy_f32(torch.from_numpy(d["x"]).to(gpu_device),
                                    torch.from_numpy(t).to(gpu_device), plan=p).cpu().numpy()
        assert np.isnan(loss[0]) and np.isnan(loss[1]) and np.isnan(loss[4])
        assert_close(loss[[2, 3, 5]], oracle.cross_entropy(d["x"], t)[[2, 3, 5]], "ce valid rows")


@pytest.mark.parametrize("bf16,cols", [(False, 257), (False, 4103), (False, 70001),
                                       (True, 257), (True, 4104), (True, 70008)])
def test_cross_entropy_out_of_range_targets_every_path(gpu_device, bf16, cols):
    """A target outside [0, cols) gives loss NaN and leaves the other rows
    within tolerance of the oracle on every path: each register and packed
    plan, the streaming plans and the split plans, float and bfloat16 rows.
    The kernels read the target logit from an in-row position whatever the
    target, and replace it by NaN where the loss is formed."""
    import torch
    t = np.array([-1, cols, 0, cols - 1, 1 << 30, 5, -(1 << 31)], np.int32)
    bad = np.array([True, True, False, False, True, False, True])
    rows = len(t)
    name = "cross_entropy_bf16" if bf16 else "cross_entropy"
    if bf16:
        x = workloads.family_inputs_bf16(rows, cols, seed=26 + cols)["x"]
        ref = oracle.cross_entropy_bf16(x, t)
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(gpu_device).view(torch.bfloat16)
        call = rr.cross_entropy_bf16
    else:
        x = workloads.family_inputs(rows, cols, seed=26 + cols)["x"]
        ref = oracle.cross_entropy(x, t)
        xd = torch.from_numpy(x).to(gpu_device)
        call = rr.cross_entropy_f32
    assert np.isnan(ref[bad]).all() and np.isfinite(ref[~bad]).all()
    td = torch.from_numpy(t).to(gpu_device)
    cands = [(p, None) for p in [None] + plans.candidate_plans(name, rows, cols)]
    for v in ((8, 4, 1) if bf16 else (4, 1)):
        for block in (256, 1024):
            lp = rr.rr_plan(2, block, block, 1, v, 0)
            if rr.rr_check_plan(name, rows, cols, lp) == 0:
                cands.append((lp, None))
    for lanes, slots in ((64, 16), (256, 16), (1024, 32)):
        sp = rr.rr_plan(3, lanes, lanes, 1, 8 if bf16 else 4, slots, 2)
        if rr.rr_check_plan(name, rows, cols, sp) == 0:
            cands.append((sp, torch.empty(rr.rr_workspace_bytes(name, rows, cols, sp), dtype=torch.uint8,
                                          device=gpu_device)))
    if cols > 65536:
        assert any(ws is not None for _, ws in cands), "no split plan at this width"
        assert any(p is not None and p.path == 2 for p, _ in cands), "no streaming plan at this width"
    for p, ws in cands:
        what = f"{name} {rows}x{cols} bad targets " + ("selected" if p is None else plans.plan_key(p))
        announce(what)
        loss = call(xd, td, plan=p, workspace=ws).cpu().numpy()
        assert np.isnan(loss[bad]).all(), f"{what}: {loss[bad]}"
        assert_close(loss[~bad], ref[~bad], what)


@pytest.mark.parametrize("op", ["softmax", "cross_entropy"])
@pytest.mark.parametrize("cols", [31, 129, 4103, 40000, 70001])
def test_masked_entries_every_plan(gpu_device, op, cols):
    """-inf entries (masked positions) add exactly 0 to the row's sum of
    exponentials and get probability 0; a row masked but for one entry puts
    all its mass there; a fully masked row is NaN throughout, as in the
    oracle. Every legal plan, the streaming plans with kept register chunks
    (masked and missing columns inside them) and the split plans."""
    import torch
    rows = 6
    a = family_host_inputs(op, rows, cols, seed=41 + cols)
    x = a["x"]
    rng = np.random.default_rng(cols)
    x[0, rng.random(cols) < 0.3] = -np.inf
    x[1, :] = -np.inf
    x[1, cols // 2] = 0.5
    x[2, :] = -np.inf
    x[3, : cols // 2] = -np.inf
    x[4, cols // 2 + 1:] = -np.inf
    if op == "cross_entropy":
        t = a["targets"]
        t[0] = int(np.flatnonzero(np.isfinite(x[0]))[0])
        t[1] = cols // 2
        t[3] = cols - 1
        t[4] = 0
    ref = run_oracle(op, a)
    assert np.isnan(ref["y" if op == "softmax" else "loss"][2]).all()
    d = to_dev(a, gpu_device)
    cands = plans.candidate_plans(op, rows, cols)
    for v in (1, 2, 4):
        for block in (256, 1024):
            for kept in (0, 32, 64, 96):
                lp = rr.rr_plan(2, block, block, 1, v, kept)
                if rr.rr_check_plan(op, rows, cols, lp) == 0:
                    cands.append(lp)
    for p in cands:
        what = f"masked {op} {rows}x{cols} {plans.plan_key(p)}"
        announce(what)
        compare(op, run_gpu(op, d, plan=p), ref, what)
    for lanes, slots in ((64, 16), (256, 16), (1024, 32)):
        sp = rr.rr_plan(3, lanes, lanes, 1, 4, slots, 2)
        if rr.rr_check_plan(op, rows, cols, sp) != 0:
            continue
        ws = torch.empty(rr.rr_workspace_bytes(op, rows, cols, sp), dtype=torch.uint8, device=gpu_device)
        what = f"masked {op} {rows}x{cols} split w{lanes} k{slots}"
        announce(what)
        if op == "softmax":
            got = {"y": rr.softmax_f32(d["x"], plan=sp, workspace=ws)}
        else:
            got = {"loss": rr.cross_entropy_f32(d["x"], d["targets"], plan=sp, workspace=ws)}
        compare(op, got, ref, what)


def test_cross_entropy_matches_softmax(gpu_device):
    import torch
    d = workloads.family_inputs(64, 4096, seed=26)
    xd = torch.from_numpy(d["x"]).to(gpu_device)
    announce("cross entropy vs softmax")
    loss = rr.cross_entropy_f32(xd, torch.from_numpy(d["targets"]).to(gpu_device)).cpu().numpy()
    p = rr.softmax_f32(xd).cpu().numpy()[np.arange(64), d["targets"]].astype(np.float64)
    assert np.all(np.abs(loss + np.log(p)) <= 1e-5 + 1e-5 * np.abs(loss))


def test_residual_layernorm_without_h_out(gpu_device):
    a = family_host_inputs("residual_layernorm", 64, 4096, seed=27)
    ref = run_oracle("residual_layernorm", a)
    announce("residual layernorm without h_out")
    got = run_gpu("residual_layernorm", to_dev(a, gpu_device), with_h=False)
    compare("residual_layernorm", got, ref, "rln no h")


def test_layernorm_constant_rows_give_beta(gpu_device):
    import torch
    d = workloads.family_inputs(3, 4096, seed=28)
    x = np.full((3, 4096), 0.75, np.float32)
    announce("layernorm constant rows")
    y = rr.layernorm_f32(torch.from_numpy(x).to(gpu_device), torch.from_numpy(d["gamma"]).to(gpu_device),
                         torch.from_numpy(d["beta"]).to(gpu_device), 1e-5).cpu().numpy()
    assert_close(y, np.broadcast_to(d["beta"], y.shape), "layernorm constant")


def test_zero_rows_is_noop(gpu_device):
    import torch
    x = torch.empty((0, 64), dtype=torch.float32, device=gpu_device)
    w = torch.ones(64, dtype=torch.float32, device=gpu_device)
    announce("zero rows")
    assert rr.rmsnorm_f32(x, w, 1e-6).shape == (0, 64)
    assert rr.row_sum_f32(x).shape == (0,)


def test_offset_views_dword_aligned(gpu_device):
    """Operands starting 4 bytes into an allocation (odd-width row origins)."""
    import torch
    wl = workloads.rmsnorm_workload(17, 257, seed=29)
    buf = torch.zeros(17 * 257 + 1, dtype=torch.float32, device=gpu_device)
    x = buf[1:].view(17, 257)
    x.copy_(torch.from_numpy(wl.x))
    wbuf = torch.zeros(258, dtype=torch.float32, device=gpu_device)
    w = wbuf[1:]
    w.copy_(torch.from_numpy(wl.w))
    announce("rmsnorm offset views")
    for p in [None] + plans.candidate_plans("rmsnorm", 17, 257):
        y = rr.rmsnorm_f32(x, w, wl.eps, plan=p)
        assert_close(y.cpu().numpy(), oracle.rmsnorm(wl.x, wl.w, wl.eps), "offset views")


def test_determinism_repeated_launches(gpu_device):
    """Fixed reduction order, no atomics: repeated launches are bit-identical."""
    import torch
    for op in OPS:
        a = family_host_inputs(op, 1024, 4096, seed=30)
        d = to_dev(a, gpu_device)
        announce(f"determinism {op}")
        first = {k: v.clone() for k, v in run_gpu(op, d, with_h=True).items()}
        for _ in range(20):
            again = run_gpu(op, d, with_h=True)
            for k in first:
                assert torch.equal(first[k].view(torch.int32), again[k].view(torch.int32)), op

"""GPU parity for the bfloat16-storage entry points against the CPU oracle.

Both sides widen the same bfloat16 inputs exactly; the GPU reduces in float
and rounds each output once from its float result, the oracle computes in
float64 and rounds once from the exact value. Element outputs must therefore
agree within one bfloat16 unit in the last place of the oracle's value (plus
1e-5 absolute); per-row outputs (row sum, loss) are float32 and keep the
float tolerance |err| <= 1e-5 + 1e-5 |ref|; h_out of residual LayerNorm is a
single rounding of the same sum on both sides and must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import plans, workloads

from parity_util import announce, assert_close

pytestmark = pytest.mark.gpu

BASE_OPS = ["rmsnorm", "sum", "softmax", "layernorm", "residual_layernorm", "cross_entropy"]
MATRIX_N = (1, 31, 33, 127, 128, 129, 257, 264, 4103, 4104)


def to_dev_bf16(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def from_dev_bf16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(bits):
    v = np.abs(oracle.bf16_to_float(bits).astype(np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -133)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -133)


def assert_bf16_close(got_bits, ref_bits, what):
    g = oracle.bf16_to_float(got_bits).astype(np.float64)
    r = oracle.bf16_to_float(ref_bits).astype(np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN pattern differs"
    ok = np.isnan(r) | (np.abs(g - r) <= bf16_ulp(ref_bits) + 1e-5)
    if not ok.all():
        i = int(np.flatnonzero(~ok.reshape(-1))[0])
        raise AssertionError(f"{what}: {int((~ok).sum())}/{ok.size} elements beyond one bf16 ulp; "
                             f"first got {g.reshape(-1)[i]!r} oracle {r.reshape(-1)[i]!r}")


def host_bf16(rows, cols, seed):
    return workloads.family_inputs_bf16(rows, cols, seed)


def run_oracle(op, d, eps):
    if op == "rmsnorm":
        return {"y": oracle.rmsnorm_bf16(d["x"], d["gamma"], eps)}
    if op == "sum":
        return {"out": oracle.row_sum_bf16(d["x"])}
    if op == "softmax":
        return {"y": oracle.softmax_bf16(d["x"])}
    if op == "layernorm":
        return {"y": oracle.layernorm_bf16(d["x"], d["gamma"], d["beta"], eps)}
    if op == "residual_layernorm":
        y, h = oracle.residual_layernorm_bf16(d["x"], d["residual"], d["gamma"], d["beta"], eps)
        return {"y": y, "h": h}
    return {"loss": oracle.cross_entropy_bf16(d["x"], d["targets"])}


def run_gpu(op, t, eps, plan=None):
    import torch
    if op == "rmsnorm":
        return {"y": rr.rmsnorm_bf16(t["x"], t["gamma"], eps, plan=plan)}
    if op == "sum":
        return {"out": rr.row_sum_bf16(t["x"], plan=plan)}
    if op == "softmax":
        return {"y": rr.softmax_bf16(t["x"], plan=plan)}
    if op == "layernorm":
        return {"y": rr.layernorm_bf16(t["x"], t["gamma"], t["beta"], eps, plan=plan)}
    if op == "residual_layernorm":
        h = torch.empty_like(t["x"])
        y = rr.residual_layernorm_bf16(t["x"], t["residual"], t["gamma"], t["beta"], eps, h_out=h, plan=plan)
        return {"y": y, "h": h}
    return {"loss": rr.cross_entropy_bf16(t["x"], t["targets"], plan=plan)}


def dev_inputs(d, device):
    import torch
    return {k: (torch.from_numpy(v).to(device) if k == "targets" else to_dev_bf16(v, device))
            for k, v in d.items()}


def compare(got, ref, what):
    for k, r in ref.items():
        if k in ("out", "loss"):
            assert_close(got[k].cpu().numpy(), r, f"{what} [{k}]")
        elif k == "h":
            assert np.array_equal(from_dev_bf16(got[k]), r), f"{what}: h_out not bit-exact"
        else:
            assert_bf16_close(from_dev_bf16(got[k]), r, f"{what} [{k}]")


def eps_of(op):
    return workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_rmsnorm_bf16_configs_full_size(gpu_device, k):
    for wl in workloads.config_workloads(k):
        x, w = workloads.as_bf16_bits(wl.x), workloads.as_bf16_bits(wl.w)
        announce(f"rmsnorm_bf16 config {k} {wl.rows}x{wl.cols} plan={rr.rr_select_plan('rmsnorm_bf16', wl.rows, wl.cols)}")
        ref = oracle.rmsnorm_bf16(x, w, wl.eps)
        y = rr.rmsnorm_bf16(to_dev_bf16(x, gpu_device), to_dev_bf16(w, gpu_device), wl.eps)
        assert_bf16_close(from_dev_bf16(y), ref, f"rmsnorm_bf16 {wl.name}")


@pytest.mark.parametrize("shape", workloads.FAMILY_SHAPES)
@pytest.mark.parametrize("op", BASE_OPS[1:])
def test_family_bf16_full_size(gpu_device, op, shape):
    rows, cols = shape
    announce(f"family {op}_bf16 {rows}x{cols} plan={rr.rr_select_plan(op + '_bf16', rows, cols)}")
    d = host_bf16(rows, cols, seed=1005)
    compare(run_gpu(op, dev_inputs(d, gpu_device), eps_of(op)), run_oracle(op, d, eps_of(op)),
            f"{op}_bf16 {rows}x{cols}")


@pytest.mark.parametrize("op", BASE_OPS)
@pytest.mark.parametrize("cols", MATRIX_N)
def test_bf16_every_legal_plan_on_ragged_matrix(gpu_device, op, cols):
    for rows in (1, 5):
        d = host_bf16(rows, cols, seed=70 + cols)
        ref = run_oracle(op, d, eps_of(op))
        t = dev_inputs(d, gpu_device)
        for p in plans.candidate_plans(op + "_bf16", rows, cols):
            what = f"{op}_bf16 {rows}x{cols} {plans.plan_key(p)}"
            announce(what)
            compare(run_gpu(op, t, eps_of(op), plan=p), ref, what)


@pytest.mark.parametrize("op", BASE_OPS)
@pytest.mark.parametrize("cols", [4096, 32776, 100000])
def test_bf16_cache_policies_and_streaming_path(gpu_device, op, cols):
    import torch
    rows = 3
    d = host_bf16(rows, cols, seed=91)
    ref = run_oracle(op, d, eps_of(op))
    t = dev_inputs(d, gpu_device)
    cands = [p for p in plans.candidate_plans(op + "_bf16", rows, cols) if p.v == 8 or p.path == 2]
    for p in cands[::2]:
        outs = []
        for cache in (0, 1, 2):
            q = rr.rr_plan.from_dict({**p.as_dict(), "cache": cache})
            what = f"{op}_bf16 {rows}x{cols} {plans.plan_key(q)}"
            announce(what)
            got = run_gpu(op, t, eps_of(op), plan=q)
            compare(got, ref, what)
            outs.append({k: v.clone() for k, v in got.items()})
        for o in outs[1:]:
            for k in o:
                a, b = o[k], outs[0][k]
                assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                                   b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (op, k)


def test_bf16_offset_views_use_narrower_packs(gpu_device):
    """Operands 2 bytes into an allocation: the selector drops to V = 1 and
    the results still match; an explicit wider plan is refused."""
    import torch
    rows, cols = 17, 256
    d = host_bf16(rows, cols, seed=92)
    ref = oracle.rmsnorm_bf16(d["x"], d["gamma"], 1e-6)
    xb = torch.zeros(rows * cols + 1, dtype=torch.bfloat16, device=gpu_device)
    x = xb[1:].view(rows, cols)
    x.copy_(to_dev_bf16(d["x"], gpu_device))
    wb = torch.zeros(cols + 1, dtype=torch.bfloat16, device=gpu_device)
    w = wb[1:]
    w.copy_(to_dev_bf16(d["gamma"], gpu_device))
    announce("rmsnorm_bf16 offset views")
    y = rr.rmsnorm_bf16(x, w, 1e-6)
    assert_bf16_close(from_dev_bf16(y), ref, "offset views")
    wide = rr.rr_plan(1, 64, 64, 1, 4, 4, 0)
    with pytest.raises(rr.RowRedError):
        rr.rmsnorm_bf16(x, w, 1e-6, plan=wide)


def test_bf16_rmsnorm_unit_magnitude_bitwise(gpu_device):
    rng = np.random.default_rng(93)
    x = workloads.as_bf16_bits(np.where(rng.random((5, 4096)) < 0.5, -1.0, 1.0).astype(np.float32))
    w = workloads.as_bf16_bits(np.ones(4096, np.float32))
    announce("rmsnorm_bf16 +-1")
    y = rr.rmsnorm_bf16(to_dev_bf16(x, gpu_device), to_dev_bf16(w, gpu_device), 0.0)
    assert np.array_equal(from_dev_bf16(y), x)


def test_bf16_row_sum_integer_rows_exact(gpu_device):
    rng = np.random.default_rng(94)
    xf = rng.integers(-100, 100, size=(64, 4096)).astype(np.float32)   # exact in bfloat16
    x = workloads.as_bf16_bits(xf)
    announce("row_sum_bf16 integers")
    out = rr.row_sum_bf16(to_dev_bf16(x, gpu_device)).cpu().numpy()
    assert np.array_equal(out, xf.astype(np.int64).sum(axis=1).astype(np.float32))


@pytest.mark.parametrize("op", ["softmax", "cross_entropy"])
@pytest.mark.parametrize("cols", [31, 129, 4104, 40000, 70000])
def test_bf16_masked_entries_every_plan(gpu_device, op, cols):
    """bfloat16 -inf entries (masked positions) on every legal plan, the
    streaming plans with kept chunks and the split plans: probability 0 where
    masked, all mass on a lone survivor, NaN for a fully masked row (as the
    oracle gives)."""
    import torch
    rows = 6
    d = host_bf16(rows, cols, seed=43 + cols)
    x = d["x"]
    neg_inf = np.uint16(0xFF80)
    rng = np.random.default_rng(cols)
    x[0, rng.random(cols) < 0.3] = neg_inf
    x[1, :] = neg_inf
    x[1, cols // 2] = np.uint16(0x3F00)          # 0.5
    x[2, :] = neg_inf
    x[3, : cols // 2] = neg_inf
    x[4, cols // 2 + 1:] = neg_inf
    if op == "cross_entropy":
        t = d["targets"]
        t[0] = int(np.flatnonzero(x[0] != neg_inf)[0])
        t[1] = cols // 2
        t[3] = cols - 1
        t[4] = 0
    ref = run_oracle(op, d, eps_of(op))
    tdev = dev_inputs(d, gpu_device)
    name = op + "_bf16"
    cands = plans.candidate_plans(name, rows, cols)
    for v in (1, 2, 4, 8):
        for block in (256, 1024):
            for kept in (0, 32, 64, 96):
                lp = rr.rr_plan(2, block, block, 1, v, kept)
                if rr.rr_check_plan(name, rows, cols, lp) == 0:
                    cands.append(lp)
    for p in cands:
        what = f"masked {name} {rows}x{cols} {plans.plan_key(p)}"
        announce(what)
        compare(run_gpu(op, tdev, eps_of(op), plan=p), ref, what)
    for lanes, slots in ((64, 16), (256, 16), (1024, 32)):
        sp = rr.rr_plan(3, lanes, lanes, 1, 8, slots, 2)
        if rr.rr_check_plan(name, rows, cols, sp) != 0:
            continue
        ws = torch.empty(rr.rr_workspace_bytes(name, rows, cols, sp), dtype=torch.uint8, device=gpu_device)
        what = f"masked {name} {rows}x{cols} split w{lanes} k{slots}"
        announce(what)
        if op == "softmax":
            got = {"y": rr.softmax_bf16(tdev["x"], plan=sp, workspace=ws)}
        else:
            got = {"loss": rr.cross_entropy_bf16(tdev["x"], tdev["targets"], plan=sp, workspace=ws)}
        compare(got, ref, what)


@pytest.mark.parametrize("op,v,slots,cols", [
    ("layernorm", 8, 32, 32776), ("layernorm", 8, 32, 65536), ("layernorm", 8, 32, 106496), ("layernorm", 8, 32, 128256),
    ("layernorm", 4, 32, 32776), ("layernorm", 4, 32, 106496), ("layernorm", 4, 32, 110000),
    ("residual_layernorm", 8, 32, 32776), ("residual_layernorm", 8, 32, 106496), ("residual_layernorm", 8, 32, 128256),
    ("softmax", 8, 64, 65544), ("softmax", 8, 64, 131072), ("softmax", 8, 64, 139264), ("softmax", 8, 64, 140000),
    ("softmax", 8, 96, 98312), ("softmax", 8, 96, 131072), ("softmax", 8, 96, 140000),
    ("rmsnorm", 8, 64, 65536), ("rmsnorm", 8, 64, 65544), ("rmsnorm", 8, 64, 139264), ("rmsnorm", 8, 64, 150000)])
def test_bf16_lds_kept_chunks(gpu_device, op, v, slots, cols):
    """1024-lane streaming plans that keep values past the register-kept ones
    in LDS, 72 per lane for bfloat16 rows: raw 16-byte packs loaded straight
    from memory (v = 8 with one input row) or bfloat16 pairs written from
    registers (residual LayerNorm's h, v = 4; 32 beside softmax's 96
    register slots). Shapes with no LDS chunk, the first one partly filled, LDS
    exactly full, and chunks streamed past it; one row offset by a large
    mean (LayerNorm statistics of shifted values), one ramp, the rest the
    standard recipe."""
    rows = 4
    d = host_bf16(rows, cols, seed=500 + cols)
    xf = oracle.bf16_to_float(d["x"]).astype(np.float32)
    xf[1] = xf[1] * 0.01 + 300.0
    xf[2] = np.linspace(-8.0, 8.0, cols, dtype=np.float32)
    d["x"] = workloads.as_bf16_bits(xf)
    ref = run_oracle(op, d, eps_of(op))
    t = dev_inputs(d, gpu_device)
    p = rr.rr_plan(2, 1024, 1024, 1, v, slots, 2)
    assert rr.rr_check_plan(op + "_bf16", rows, cols, p) == 0
    what = f"lds-kept {op}_bf16 {rows}x{cols} v{v} k{slots}"
    announce(what)
    compare(run_gpu(op, t, eps_of(op), plan=p), ref, what)

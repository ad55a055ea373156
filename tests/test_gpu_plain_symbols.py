"""The plain C entry points themselves — rmsnorm_f32(x, w, y, rows, cols, eps,
stream) and its five siblings, and the six bfloat16 forms — called through
ctypes with raw device pointers and the HIP stream handle (no binding code in
between), compared element by element with the CPU oracle on the measured
configurations and a ragged shape."""
import ctypes

import numpy as np
import pytest

import oracle
from row_reduction_amd import _capi, workloads

from parity_util import announce, assert_close
from test_gpu_bf16 import assert_bf16_close, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

RMSNORM_CASES = [(1, 127, 0.0), (17, 257, 0.0), (64, 4096, 0.01), (1024, 4096, 0.0), (5, 4103, 0.0)]
FAMILY_CASES = list(workloads.FAMILY_SHAPES) + [(5, 4103), (3, 40000)]
FAMILY_OPS = ["sum", "softmax", "layernorm", "residual_layernorm", "cross_entropy"]


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _sync_ok(name, status):
    import torch
    assert status == _capi.RR_OK, f"{name} returned {_capi.status_string(status)}"
    torch.cuda.synchronize()


@pytest.mark.parametrize("rows,cols,outliers", RMSNORM_CASES)
def test_rmsnorm_f32_symbol(gpu_device, rows, cols, outliers):
    import torch
    L = _capi.lib()
    wl = workloads.rmsnorm_workload(rows, cols, seed=3000 + cols, outlier_fraction=outliers)
    x = torch.from_numpy(wl.x).to(gpu_device)
    w = torch.from_numpy(wl.w).to(gpu_device)
    y = torch.full_like(x, float("nan"))
    announce(f"rmsnorm_f32 symbol {rows}x{cols}")
    _sync_ok("rmsnorm_f32", L.rmsnorm_f32(_p(x), _p(w), _p(y), rows, cols, wl.eps, _stream()))
    assert_close(y.cpu().numpy(), oracle.rmsnorm(wl.x, wl.w, wl.eps), f"rmsnorm_f32 {rows}x{cols}")


def _family_f32(L, op, t, rows, cols, eps):
    """Calls the plain float entry point of `op`; returns the output tensors."""
    import torch
    s = _stream()
    if op == "sum":
        out = torch.full((rows,), float("nan"), device=t["x"].device)
        _sync_ok(op, L.row_sum_f32(_p(t["x"]), _p(out), rows, cols, s))
        return {"out": out}
    if op == "softmax":
        y = torch.full_like(t["x"], float("nan"))
        _sync_ok(op, L.softmax_f32(_p(t["x"]), _p(y), rows, cols, s))
        return {"y": y}
    if op == "layernorm":
        y = torch.full_like(t["x"], float("nan"))
        _sync_ok(op, L.layernorm_f32(_p(t["x"]), _p(t["gamma"]), _p(t["beta"]), _p(y), rows, cols, eps, s))
        return {"y": y}
    if op == "residual_layernorm":
        y = torch.full_like(t["x"], float("nan"))
        h = torch.full_like(t["x"], float("nan"))
        _sync_ok(op, L.residual_layernorm_f32(_p(t["x"]), _p(t["residual"]), _p(t["gamma"]), _p(t["beta"]),
                                              _p(y), _p(h), rows, cols, eps, s))
        return {"y": y, "h": h}
    loss = torch.full((rows,), float("nan"), device=t["x"].device)
    _sync_ok(op, L.cross_entropy_f32(_p(t["x"]), _p(t["targets"]), _p(loss), rows, cols, s))
    return {"loss": loss}


def _family_oracle(op, d, eps):
    if op == "sum":
        return {"out": oracle.row_sum(d["x"])}
    if op == "softmax":
        return {"y": oracle.softmax(d["x"])}
    if op == "layernorm":
        return {"y": oracle.layernorm(d["x"], d["gamma"], d["beta"], eps)}
    if op == "residual_layernorm":
        y, h = oracle.residual_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], eps)
        return {"y": y, "h": h}
    return {"loss": oracle.cross_entropy(d["x"], d["targets"])}


@pytest.mark.parametrize("shape", FAMILY_CASES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("op", FAMILY_OPS)
def test_family_f32_symbol(gpu_device, op, shape):
    import torch
    rows, cols = shape
    L = _capi.lib()
    d = workloads.family_inputs(rows, cols, seed=3100 + cols)
    t = {k: torch.from_numpy(v).to(gpu_device) for k, v in d.items()}
    eps = workloads.LAYERNORM_EPS
    announce(f"{op}_f32 symbol {rows}x{cols}")
    got = _family_f32(L, op, t, rows, cols, eps)
    for k, r in _family_oracle(op, d, eps).items():
        g = got[k].cpu().numpy()
        if k == "h":
            assert np.array_equal(g.view(np.int32), r.view(np.int32)), f"{op} {rows}x{cols}: h_out not bit-exact"
        else:
            assert_close(g, r, f"{op}_f32 symbol {rows}x{cols} [{k}]")


BF16_OPS = ["rmsnorm"] + FAMILY_OPS


@pytest.mark.parametrize("shape", [(1, 127), (17, 257), (64, 4096), (1024, 4096), (5, 4104)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("op", BF16_OPS)
def test_bf16_symbol(gpu_device, op, shape):
    import torch
    rows, cols = shape
    L = _capi.lib()
    d = workloads.family_inputs_bf16(rows, cols, seed=3200 + cols)
    eps = workloads.RMSNORM_EPS if op == "rmsnorm" else workloads.LAYERNORM_EPS
    t = {k: (torch.from_numpy(v).to(gpu_device) if k == "targets" else to_dev_bf16(v, gpu_device))
         for k, v in d.items()}
    s = _stream()
    empty = lambda: torch.full_like(t["x"], float("nan"))
    announce(f"{op}_bf16 symbol {rows}x{cols}")
    if op == "rmsnorm":
        y = empty()
        _sync_ok(op, L.rmsnorm_bf16(_p(t["x"]), _p(t["gamma"]), _p(y), rows, cols, eps, s))
        got, ref = {"y": y}, {"y": oracle.rmsnorm_bf16(d["x"], d["gamma"], eps)}
    elif op == "sum":
        out = torch.full((rows,), float("nan"), device=gpu_device)
        _sync_ok(op, L.row_sum_bf16(_p(t["x"]), _p(out), rows, cols, s))
        got, ref = {"out": out}, {"out": oracle.row_sum_bf16(d["x"])}
    elif op == "softmax":
        y = empty()
        _sync_ok(op, L.softmax_bf16(_p(t["x"]), _p(y), rows, cols, s))
        got, ref = {"y": y}, {"y": oracle.softmax_bf16(d["x"])}
    elif op == "layernorm":
        y = empty()
        _sync_ok(op, L.layernorm_bf16(_p(t["x"]), _p(t["gamma"]), _p(t["beta"]), _p(y), rows, cols, eps, s))
        got, ref = {"y": y}, {"y": oracle.layernorm_bf16(d["x"], d["gamma"], d["beta"], eps)}
    elif op == "residual_layernorm":
        y, h = empty(), empty()
        _sync_ok(op, L.residual_layernorm_bf16(_p(t["x"]), _p(t["residual"]), _p(t["gamma"]), _p(t["beta"]),
                                               _p(y), _p(h), rows, cols, eps, s))
        yr, hr = oracle.residual_layernorm_bf16(d["x"], d["residual"], d["gamma"], d["beta"], eps)
        got, ref = {"y": y, "h": h}, {"y": yr, "h": hr}
    else:
        loss = torch.full((rows,), float("nan"), device=gpu_device)
        _sync_ok(op, L.cross_entropy_bf16(_p(t["x"]), _p(t["targets"]), _p(loss), rows, cols, s))
        got, ref = {"loss": loss}, {"loss": oracle.cross_entropy_bf16(d["x"], d["targets"])}
    for k, r in ref.items():
        if k in ("out", "loss"):
            assert_close(got[k].cpu().numpy(), r, f"{op}_bf16 symbol {rows}x{cols} [{k}]")
        elif k == "h":
            assert np.array_equal(from_dev_bf16(got[k]), r), f"{op}_bf16 {rows}x{cols}: h_out not bit-exact"
        else:
            assert_bf16_close(from_dev_bf16(got[k]), r, f"{op}_bf16 symbol {rows}x{cols} [{k}]")

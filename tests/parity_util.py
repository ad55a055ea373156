"""Shared helpers for the GPU parity tests: run one operator through the C ABI
on the GPU and through the CPU oracle on the same inputs, compare every
element of every output."""
from __future__ import annotations

import sys

import numpy as np

import oracle

RTOL = 1e-5
ATOL = 1e-5


def assert_close(got, ref, what: str) -> None:
    """|got - ref| <= ATOL + RTOL * |ref| for every element (NaN must match NaN)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        worst = int(np.argmax(err / bound))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside |err| <= 1e-5 + 1e-5|ref|; "
            f"first bad got {g[i]!r} oracle {r[i]!r}; worst ratio {float((err / bound)[worst]):.3f}")


def announce(msg: str) -> None:
    """Name the case on stdout before its GPU work, flushed."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arrays: dict, device):
    import torch
    return {k: (torch.from_numpy(np.ascontiguousarray(v)).to(device) if isinstance(v, np.ndarray) else v)
            for k, v in arrays.items()}


def run_gpu(op: str, d: dict, plan=None, with_h=False, out=None):
    """Run `op` on device tensors `d` (x, w, beta, residual, targets, eps)."""
    import row_reduction_amd as rr
    if op == "rmsnorm":
        return {"y": rr.rmsnorm_f32(d["x"], d["w"], d["eps"], y=out, plan=plan)}
    if op == "sum":
        return {"out": rr.row_sum_f32(d["x"], plan=plan)}
    if op == "softmax":
        return {"y": rr.softmax_f32(d["x"], y=out, plan=plan)}
    if op == "layernorm":
        return {"y": rr.layernorm_f32(d["x"], d["w"], d["beta"], d["eps"], y=out, plan=plan)}
    if op == "residual_layernorm":
        import torch
        h = torch.empty_like(d["x"]) if with_h else None
        y = rr.residual_layernorm_f32(d["x"], d["residual"], d["w"], d["beta"], d["eps"], y=out,
                                      h_out=h, plan=plan)
        res = {"y": y}
        if with_h:
            res["h"] = h
        return res
    if op == "cross_entropy":
        return {"loss": rr.cross_entropy_f32(d["x"], d["targets"], plan=plan)}
    raise ValueError(op)


def run_oracle(op: str, a: dict) -> dict:
    if op == "rmsnorm":
        return {"y": oracle.rmsnorm(a["x"], a["w"], a["eps"])}
    if op == "sum":
        return {"out": oracle.row_sum(a["x"])}
    if op == "softmax":
        return {"y": oracle.softmax(a["x"])}
    if op == "layernorm":
        return {"y": oracle.layernorm(a["x"], a["w"], a["beta"], a["eps"])}
    if op == "residual_layernorm":
        y, h = oracle.residual_layernorm(a["x"], a["residual"], a["w"], a["beta"], a["eps"])
        return {"y": y, "h": h}
    if op == "cross_entropy":
        return {"loss": oracle.cross_entropy(a["x"], a["targets"])}
    raise ValueError(op)


def host_inputs(op: str, x, w=None, beta=None, residual=None, targets=None, eps=None) -> dict:
    from row_reduction_amd import workloads
    a = {"x": x}
    if op == "rmsnorm":
        a["w"], a["eps"] = w, workloads.RMSNORM_EPS if eps is None else eps
    if op in ("layernorm", "residual_layernorm"):
        a["w"], a["beta"] = w, beta
        a["eps"] = workloads.LAYERNORM_EPS if eps is None else eps
    if op == "residual_layernorm":
        a["residual"] = residual
    if op == "cross_entropy":
        a["targets"] = targets
    return a


def family_host_inputs(op: str, rows: int, cols: int, seed: int) -> dict:
    from row_reduction_amd import workloads
    d = workloads.family_inputs(rows, cols, seed)
    return host_inputs(op, d["x"], w=d["gamma"], beta=d["beta"], residual=d["residual"],
                       targets=d["targets"])


def compare(op: str, got: dict, ref: dict, what: str, bitwise_h: bool = True) -> None:
    for k, r in ref.items():
        if k not in got:
            continue
        g = got[k].cpu().numpy()
        if k == "h" and bitwise_h:
            assert np.array_equal(g.view(np.int32), r.view(np.int32)), f"{what}: h_out not bit-exact"
        else:
            assert_close(g, r, f"{what} [{k}]")

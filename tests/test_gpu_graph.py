"""HIP-graph capture of the entry points: each operator is captured once and
replayed several times, with new inputs copied in and eager work and
synchronisations between replays; every replay must equal the eager call on
the same inputs bit for bit (the library records only kernel launches, no
memset nodes)."""
import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import workloads

from parity_util import announce

pytestmark = pytest.mark.gpu


def _call(op, t):
    if op == "rmsnorm":
        return rr.rmsnorm_f32(t["x"], t["gamma"], 1e-6, y=t["y"])
    if op == "sum":
        return rr.row_sum_f32(t["x"], out=t["rowout"])
    if op == "softmax":
        return rr.softmax_f32(t["x"], y=t["y"])
    if op == "layernorm":
        return rr.layernorm_f32(t["x"], t["gamma"], t["beta"], 1e-5, y=t["y"])
    if op == "residual_layernorm":
        return rr.residual_layernorm_f32(t["x"], t["residual"], t["gamma"], t["beta"], 1e-5,
                                         y=t["y"], h_out=t["h"])
    return rr.cross_entropy_f32(t["x"], t["targets"], loss=t["rowout"])


@pytest.mark.parametrize("shape", [(17, 257), (1024, 4096), (3, 40000)])
@pytest.mark.parametrize("op", list(workloads.OPS))
def test_graph_replays_match_eager(gpu_device, op, shape):
    import torch
    rows, cols = shape
    announce(f"graph {op} {rows}x{cols}")
    inputs = [workloads.family_inputs(rows, cols, seed=40 + i) for i in range(4)]
    t = {k: torch.from_numpy(v).to(gpu_device) for k, v in inputs[0].items()}
    t["y"] = torch.empty_like(t["x"])
    t["h"] = torch.empty_like(t["x"])
    t["rowout"] = torch.empty(rows, dtype=torch.float32, device=gpu_device)
    out_keys = ["rowout"] if op in ("sum", "cross_entropy") else (["y", "h"] if op == "residual_layernorm" else ["y"])

    _call(op, t)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(op, t)
    torch.cuda.synchronize()

    for i, d in enumerate(inputs):
        for k, v in d.items():
            t[k].copy_(torch.from_numpy(v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = {k: t[k].clone() for k in out_keys}
        # Eager work between replays, then the eager reference on the same inputs.
        for k in out_keys:
            t[k].fill_(float("nan"))
        _call(op, t)
        torch.cuda.synchronize()
        for k in out_keys:
            assert torch.equal(replayed[k].view(torch.int32), t[k].view(torch.int32)), (op, i, k)
        assert np.isfinite(replayed[out_keys[0]].cpu().numpy()).all()

"""GPU parity at the size limits: a matrix of more than 2^31 elements (row
offsets past the int32 range) and a single row of the largest accepted
column count (RR_MAX_COLS, column indices near the int32 range). Inputs are
drawn on the device from a seeded generator; sampled rows, or sampled
columns of the one long row, are copied back and compared with the CPU
oracle (the long row through the oracle's one-row forms, whose statistic
covers the whole row)."""
import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import _capi

from parity_util import announce, assert_close

pytestmark = pytest.mark.gpu

EPS = 1e-6


def draw(torch, shape, seed, device):
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def sample_rows(rows, seed, n=56):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(4), np.arange(rows - 4, rows), rng.integers(0, rows, n)]))


def test_more_than_2_31_elements(gpu_device):
    """525288 x 4096 = 2^31 + 4 Mi elements (8.6 GB per float tensor)."""
    import torch
    rows, cols = (1 << 19) + 1000, 4096
    assert rows * cols > 2 ** 31
    x = draw(torch, (rows, cols), 11, gpu_device)
    w = (draw(torch, (cols,), 12, gpu_device).abs() * 0.5 + 0.5).contiguous()
    idx = sample_rows(rows, 13)
    ti = torch.from_numpy(idx).to(gpu_device)
    xs, wh = x[ti].cpu().numpy(), w.cpu().numpy()

    announce(f"large rmsnorm_f32 {rows}x{cols} plan={rr.rr_select_plan('rmsnorm', rows, cols).as_dict()}")
    y = rr.rmsnorm_f32(x, w, EPS)
    assert_close(y[ti].cpu().numpy(), oracle.rmsnorm(xs, wh, EPS), "rmsnorm > 2^31 elements")

    announce(f"large row_sum_f32 {rows}x{cols}")
    out = rr.row_sum_f32(x)
    assert_close(out[ti].cpu().numpy(), oracle.row_sum(xs), "row sum > 2^31 elements")

    announce(f"large softmax_f32 {rows}x{cols}")
    rr.softmax_f32(x, y=y)
    assert_close(y[ti].cpu().numpy(), oracle.softmax(xs), "softmax > 2^31 elements")
    del y, out

    announce(f"large rmsnorm_bf16 {rows}x{cols}")
    xb, wb = x.to(torch.bfloat16), w.to(torch.bfloat16)
    del x
    yb = rr.rmsnorm_bf16(xb, wb, EPS)
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.rmsnorm_bf16(bits(xb[ti]), bits(wb), EPS)
    from test_gpu_bf16 import assert_bf16_close
    assert_bf16_close(bits(yb[ti]), ref, "rmsnorm_bf16 > 2^31 elements")


def test_single_row_of_max_cols(gpu_device):
    """One row of RR_MAX_COLS = 2^31 - 2^20 columns on the streaming path
    (the split path cannot take it: it would need more than 1024 slices)."""
    import torch
    cols = _capi.RR_MAX_COLS
    assert rr.rr_workspace_bytes("rmsnorm", 1, cols) == 0
    x = draw(torch, (1, cols), 21, gpu_device)
    rng = np.random.default_rng(22)
    idx = np.unique(np.concatenate([np.arange(4096), np.arange(cols - 4096, cols),
                                    rng.integers(0, cols, 8192)]))
    ti = torch.from_numpy(idx).to(gpu_device)
    xh = x[0].cpu().numpy()

    announce(f"max-cols row_sum_f32 1x{cols} plan={rr.rr_select_plan('sum', 1, cols).as_dict()}")
    out = rr.row_sum_f32(x)
    assert_close(out.cpu().numpy(), np.array([oracle.row_sum_long(xh)]), "row sum max cols")

    announce(f"max-cols rmsnorm_f32 1x{cols} plan={rr.rr_select_plan('rmsnorm', 1, cols).as_dict()}")
    w = (draw(torch, (cols,), 23, gpu_device).abs() * 0.5 + 0.5).contiguous()
    y = rr.rmsnorm_f32(x, w, EPS)
    got = y[0][ti].cpu().numpy()
    wh = w.cpu().numpy()
    del w
    assert_close(got, oracle.rmsnorm_sampled(xh, wh, EPS, idx), "rmsnorm max cols")
    del wh

    announce(f"max-cols softmax_f32 1x{cols} plan={rr.rr_select_plan('softmax', 1, cols).as_dict()}")
    rr.softmax_f32(x, y=y)
    assert_close(y[0][ti].cpu().numpy(), oracle.softmax_sampled(xh, idx), "softmax max cols")

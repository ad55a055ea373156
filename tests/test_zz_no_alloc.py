"""rmsnorm_f32_noalloc: split rows whose partials live in the library's static
device buffer, for callers that cannot allocate. Its outputs must equal those
of rmsnorm_f32_ws (the same kernels with a caller workspace) bit for bit and
match the oracle within |err| <= 1e-5 + 1e-5 |ref|, over calls in a row on
one GPU, the later ones smaller, which find the buffer holding the earlier
call's partials."""
import ctypes

import numpy as np
import pytest

import oracle
import row_reduction_amd as rr
from row_reduction_amd import _capi, workloads
from row_reduction_amd._capi import RR_PATH_SPLIT

from parity_util import announce, assert_close


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _split_plan(lanes, slots):
    return rr.rr_plan(RR_PATH_SPLIT, lanes, lanes, 1, 4, slots, 2)


def test_noalloc_refuses_a_split_beyond_its_buffer_before_any_launch():
    """An explicit split plan whose partials exceed the static buffer is
    refused on the host (rows * slices * 16 > 1 MiB); nothing is enqueued, so
    placeholder pointers are never dereferenced."""
    L = _capi.lib()
    rows, cols = 255, 300000
    plan = _split_plan(64, 16)
    assert rr.rr_check_plan("rmsnorm", rows, cols, plan) == _capi.RR_OK
    need = rr.rr_workspace_bytes("rmsnorm", rows, cols, plan)
    assert need > _capi.RR_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = L.rmsnorm_f32_noalloc(fake, fake, fake, rows, cols, 1e-6, ctypes.byref(plan), None)
    assert st == _capi.RR_ERR_UNSUPPORTED
    st = L.rmsnorm_f32_noalloc(fake, None, fake, rows, cols, 1e-6, None, None)
    assert st == _capi.RR_ERR_INVALID_ARGUMENT
    assert L.rmsnorm_f32_noalloc(None, None, None, 0, cols, 1e-6, None, None) == _capi.RR_OK


# (rows, cols, explicit split plan or None for the selector), largest first:
# each later call finds the previous call's partials in the buffer.
CALLS = [
    (8, 1 << 20, None),
    (4, 1 << 20, _split_plan(64, 16)),        # 4 x 1024 partials
    (3, 300000, _split_plan(256, 16)),
    (2, 100003, None),
    (1, 40000, _split_plan(1024, 32)),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(gpu_device):
    import torch
    L = _capi.lib()
    for k, (rows, cols, plan) in enumerate(CALLS):
        wl = workloads.rmsnorm_workload(rows, cols, seed=4000 + k)
        x = torch.from_numpy(wl.x).to(gpu_device)
        w = torch.from_numpy(wl.w).to(gpu_device)
        sel_ws = rr.rr_workspace_bytes("rmsnorm", rows, cols, plan)
        assert 0 < sel_ws <= _capi.RR_NOALLOC_SCRATCH_BYTES, (rows, cols, sel_ws)
        ws = torch.empty(sel_ws, dtype=torch.uint8, device=gpu_device)
        y_ws = torch.full_like(x, float("nan"))
        y_na = torch.full_like(x, float("nan"))
        pp = ctypes.byref(plan) if plan is not None else None
        what = f"rmsnorm_f32_noalloc {rows}x{cols} " + (f"w{plan.lanes_per_row} k{plan.slots}" if plan else "selected")
        announce(what)
        st = L.rmsnorm_f32_ws(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                              ctypes.c_void_p(y_ws.data_ptr()), rows, cols, wl.eps, pp,
                              ctypes.c_void_p(ws.data_ptr()), sel_ws, _stream())
        assert st == _capi.RR_OK, _capi.status_string(st)
        st = L.rmsnorm_f32_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                   ctypes.c_void_p(y_na.data_ptr()), rows, cols, wl.eps, pp, _stream())
        assert st == _capi.RR_OK, _capi.status_string(st)
        torch.cuda.synchronize()
        got_ws = y_ws.cpu().numpy()
        got_na = y_na.cpu().numpy()
        assert np.array_equal(got_na.view(np.int32), got_ws.view(np.int32)), f"{what}: differs from rmsnorm_f32_ws"
        assert_close(got_na, oracle.rmsnorm(wl.x, wl.w, wl.eps), what)


@pytest.mark.gpu
def test_noalloc_binding_plain_shape(gpu_device):
    """A shape the selector does not split runs the plain plan (no buffer)."""
    import torch
    wl = workloads.rmsnorm_workload(64, 4096, seed=4100, outlier_fraction=0.01)
    x = torch.from_numpy(wl.x).to(gpu_device)
    w = torch.from_numpy(wl.w).to(gpu_device)
    announce("rmsnorm_f32_noalloc 64x4096 binding")
    y = rr.rmsnorm_f32_noalloc(x, w, wl.eps)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.rmsnorm(wl.x, wl.w, wl.eps), "noalloc 64x4096")


@pytest.mark.gpu
def test_noalloc_on_a_non_default_stream(gpu_device):
    """On a stream of its own (a non-null handle, so the buffer is found
    through the stream's device rather than the current one) the results
    equal rmsnorm_f32_ws's on that stream bit for bit."""
    import torch
    rows, cols = 4, 1 << 20
    wl = workloads.rmsnorm_workload(rows, cols, seed=4200)
    x = torch.from_numpy(wl.x).to(gpu_device)
    w = torch.from_numpy(wl.w).to(gpu_device)
    sel_ws = rr.rr_workspace_bytes("rmsnorm", rows, cols)
    assert 0 < sel_ws <= _capi.RR_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(sel_ws, dtype=torch.uint8, device=gpu_device)
    y_ws = torch.full_like(x, float("nan"))
    y_na = torch.full_like(x, float("nan"))
    torch.cuda.synchronize()
    L = _capi.lib()
    s = torch.cuda.Stream(device=gpu_device)
    announce("rmsnorm_f32_noalloc 4x1048576 on its own stream")
    with torch.cuda.stream(s):
        handle = _stream()
        assert handle.value, "expected a non-null stream handle"
        st = L.rmsnorm_f32_ws(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                              ctypes.c_void_p(y_ws.data_ptr()), rows, cols, wl.eps, None,
                              ctypes.c_void_p(ws.data_ptr()), sel_ws, handle)
        assert st == _capi.RR_OK, _capi.status_string(st)
        st = L.rmsnorm_f32_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                   ctypes.c_void_p(y_na.data_ptr()), rows, cols, wl.eps, None, handle)
        assert st == _capi.RR_OK, _capi.status_string(st)
    s.synchronize()
    got_ws = y_ws.cpu().numpy()
    got_na = y_na.cpu().numpy()
    assert np.array_equal(got_na.view(np.int32), got_ws.view(np.int32)), "differs from rmsnorm_f32_ws"
    assert_close(got_na, oracle.rmsnorm(wl.x, wl.w, wl.eps), "noalloc on its own stream")


@pytest.mark.gpu
def test_noalloc_under_graph_capture(gpu_device):
    """Captured into a HIP graph, as callers that cannot allocate use it (the
    capture stream is not the null stream; an eager call first looks the
    buffer up outside the capture): every replay, with new inputs copied in
    and eager work and synchronisations between replays, equals the eager
    rmsnorm_f32_ws call on the same inputs bit for bit."""
    import torch
    rows, cols = 4, 1 << 20
    loads = [workloads.rmsnorm_workload(rows, cols, seed=4300 + i) for i in range(3)]
    eps = loads[0].eps
    assert all(wl.eps == eps for wl in loads)
    x = torch.from_numpy(loads[0].x).to(gpu_device)
    w = torch.from_numpy(loads[0].w).to(gpu_device)
    y = torch.empty_like(x)
    announce("rmsnorm_f32_noalloc 4x1048576 under graph capture")
    rr.rmsnorm_f32_noalloc(x, w, eps, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rr.rmsnorm_f32_noalloc(x, w, eps, y)
    torch.cuda.synchronize()
    ws = torch.empty(rr.rr_workspace_bytes("rmsnorm", rows, cols), dtype=torch.uint8, device=gpu_device)
    for i, wl in enumerate(loads):
        x.copy_(torch.from_numpy(wl.x))
        w.copy_(torch.from_numpy(wl.w))
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = y.clone()
        ref = rr.rmsnorm_f32(x, w, eps, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int32), ref.view(torch.int32)), f"replay {i}"
        assert_close(replayed.cpu().numpy(), oracle.rmsnorm(wl.x, wl.w, wl.eps), f"graph replay {i}")

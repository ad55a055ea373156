"""Streams (GPU): every entry point enqueues on the stream it is given (the
binding passes torch's current stream, or an explicit one), after the work
already on that stream; and host threads driving their own streams at once
get correct results."""
import threading

import numpy as np
import pytest

import oracle
import row_reduction_amd as rr

from parity_util import announce, assert_close, compare, family_host_inputs, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu

OPS = ["rmsnorm", "sum", "softmax", "layernorm", "residual_layernorm", "cross_entropy"]


@pytest.mark.parametrize("op", OPS)
def test_current_stream_is_used(gpu_device, op):
    import torch
    a = family_host_inputs(op, 37, 3001, seed=61)
    ref = run_oracle(op, a)
    s = torch.cuda.Stream()
    announce(f"stream {op}")
    with torch.cuda.stream(s):
        d = to_dev(a, gpu_device)
        got = run_gpu(op, d, with_h=True)
    s.synchronize()
    compare(op, got, ref, f"{op} on a side stream")


def test_launch_is_ordered_after_earlier_work_on_its_stream(gpu_device):
    """A fill of x queued on a side stream, then RMSNorm on that stream with
    no synchronisation in between: the kernel must see the filled rows
    (constant c: y = w * c / sqrt(c^2 + eps))."""
    import torch
    rows, cols, c, eps = 8192, 8192, 0.75, 1e-6
    w = torch.linspace(0.5, 1.5, cols, device=gpu_device)
    x = torch.randn(rows, cols, device=gpu_device)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    announce("stream ordering")
    with torch.cuda.stream(s):
        for _ in range(3):
            x.mul_(1.0001)            # keep the stream busy before the fill
        x.fill_(c)
        y = torch.empty_like(x)
        rr.rmsnorm_f32(x, w, eps, y=y, stream=s.cuda_stream)
    s.synchronize()
    wh = w.cpu().numpy()
    ref = oracle.rmsnorm(np.full((1, cols), c, np.float32), wh, eps)[0]
    got = y.cpu().numpy()
    assert_close(got, np.broadcast_to(ref, got.shape), "rmsnorm after fill on the same stream")


def test_host_threads_on_their_own_streams(gpu_device):
    import torch
    cases = [(op, family_host_inputs(op, 64 + 7 * i, 1000 + 333 * i, seed=70 + i)) for i, op in enumerate(OPS)]
    refs = [run_oracle(op, a) for op, a in cases]
    results, errors = {}, []

    def worker(i):
        try:
            op, a = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                d = to_dev(a, gpu_device)
                outs = [run_gpu(op, d, with_h=True) for _ in range(20)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below
            errors.append(e)

    announce("threads with their own streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (op, _) in enumerate(cases):
        for k, got in enumerate(results[i]):
            compare(op, got, refs[i], f"{op} thread {i} call {k}")

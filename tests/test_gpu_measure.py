"""The measurement helpers the benchmark's ceilings and floors come from:
rr_copy_f32 and rr_stream_f32 (copy mode) must copy every element exactly
and nothing past the end, in every geometry and on ragged sizes;
rr_stream_f32's read-only mode must read and never write; rr_empty_kernel
must launch. A helper that skipped data would report a ceiling it never
reached."""
import numpy as np
import pytest

import row_reduction_amd as rr

from parity_util import announce

pytestmark = pytest.mark.gpu

SIZES = (1, 3, 4, 5, 1023, 4097, 3 * 1024 * 8 + 1, (1 << 20) + 7)
GUARD = 64


def _data(n, seed):
    return np.random.default_rng(seed).standard_normal(n).astype(np.float32)


def test_copy_kernel_every_size(gpu_device):
    import torch
    for i, n in enumerate(SIZES):
        announce(f"rr_copy_f32 n={n}")
        src = torch.from_numpy(_data(n, 70 + i)).to(gpu_device)
        buf = torch.full((n + GUARD,), float("nan"), device=gpu_device)
        rr.rr_copy_f32(src, buf[:n])
        torch.cuda.synchronize()
        out = buf.cpu().numpy()
        assert np.array_equal(out[:n].view(np.int32), src.cpu().numpy().view(np.int32)), n
        assert np.isnan(out[n:]).all(), f"rr_copy_f32 wrote past {n} elements"


@pytest.mark.parametrize("packs", [1, 2, 4, 8])
@pytest.mark.parametrize("block", [256, 512, 1024])
def test_stream_copy_every_geometry(gpu_device, packs, block):
    import torch
    for i, n in enumerate(SIZES):
        announce(f"rr_stream_f32 copy n={n} packs={packs} block={block}")
        src = torch.from_numpy(_data(n, 80 + i)).to(gpu_device)
        buf = torch.full((n + GUARD,), float("nan"), device=gpu_device)
        rr.rr_stream_f32(src, buf[:n], copy=True, packs_per_thread=packs, block=block)
        torch.cuda.synchronize()
        out = buf.cpu().numpy()
        assert np.array_equal(out[:n].view(np.int32), src.cpu().numpy().view(np.int32)), (n, packs, block)
        assert np.isnan(out[n:]).all(), f"copy wrote past {n} elements ({packs}, {block})"


@pytest.mark.parametrize("packs", [1, 8])
@pytest.mark.parametrize("block", [256, 1024])
def test_stream_read_never_writes(gpu_device, packs, block):
    import torch
    for i, n in enumerate(SIZES):
        announce(f"rr_stream_f32 read n={n} packs={packs} block={block}")
        src = torch.from_numpy(_data(n, 90 + i)).to(gpu_device)
        threads = -(-n // (4 * packs * block)) * block
        sink = torch.full((threads + GUARD,), 7.0, device=gpu_device)
        rr.rr_stream_f32(src, sink, copy=False, packs_per_thread=packs, block=block)
        torch.cuda.synchronize()
        assert (sink.cpu().numpy() == 7.0).all(), f"read-only stream wrote ({n}, {packs}, {block})"


def test_empty_kernel_launches(gpu_device):
    import torch
    from row_reduction_amd import _capi
    assert _capi.lib().rr_empty_kernel(None) == _capi.RR_OK
    torch.cuda.synchronize()

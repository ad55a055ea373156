"""The binding works whichever is imported first, the library or torch: the
library must bind to the HIP runtime torch ships (same soname), or torch's
stream handles are foreign to it and every launch fails. Run in a child
process that loads the library before anything imports torch."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
from row_reduction_amd import _capi
_capi.lib()                                # library first, torch not imported yet by the caller
import numpy as np
import torch
import row_reduction_amd as rr
import oracle
from row_reduction_amd import workloads
wl = workloads.rmsnorm_workload(64, 4096, seed=77)
x = torch.from_numpy(wl.x).cuda()
w = torch.from_numpy(wl.w).cuda()
y = rr.rmsnorm_f32(x, w, wl.eps)
torch.cuda.synchronize()
ref = oracle.rmsnorm(wl.x, wl.w, wl.eps)
err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
assert (err <= 1e-5 + 1e-5 * np.abs(ref)).all()
print("load-order ok")
"""


def test_library_loaded_before_torch(gpu_device):
    print("child: library loaded before torch, rmsnorm_f32 64x4096", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "load-order ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]

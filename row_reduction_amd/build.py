"""Build librowred.so (HIP for gfx950) in-tree.

Each translation unit compiles in its own hipcc process (in parallel), then
one link step produces ``row_reduction_amd/librowred.so``. Objects go to
``row_reduction_amd/_build/`` (not committed).

Device code is built with packed-FP32 instruction selection turned off
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is expected.

Every kernel instance must keep all its values in registers: the compiler's
resource report is read for each one, and the build fails if any instance
needs per-lane scratch memory (a spill). The report's per-instance VGPR,
scratch, LDS and occupancy figures are written to ``_build/resources.txt``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librowred.so")

ARCH = "gfx950"
HIP_SOURCES = [
    "api.hip",
    "measure.hip",
    "kernels_rmsnorm.hip",
    "kernels_row_sum.hip",
    "kernels_softmax.hip",
    "kernels_layernorm.hip",
    "kernels_residual_layernorm.hip",
    "kernels_cross_entropy.hip",
    "kernels_rmsnorm_bf16.hip",
    "kernels_row_sum_bf16.hip",
    "kernels_softmax_bf16.hip",
    "kernels_layernorm_bf16.hip",
    "kernels_residual_layernorm_bf16.hip",
    "kernels_cross_entropy_bf16.hip",
    "kernels_batch.hip",
]
CXX_SOURCES = ["plan.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librowred)")


def hip_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


RESOURCE_KEYS = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
                 "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}


def _resources(lines: list[str]) -> dict:
    """Per-kernel figures from -Rpass-analysis=kernel-resource-usage remarks."""
    out, name = {}, None
    for ln in lines:
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?): (\d+)", ln)
        if m and name and m.group(1) in RESOURCE_KEYS:
            out[name][RESOURCE_KEYS[m.group(1)]] = int(m.group(2))
    return out


def _run(cmd: list[str]) -> dict:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass's notice about the device-only feature is expected noise;
    # resource remarks are collected, not printed.
    raw = proc.stdout.splitlines()
    res = _resources(raw)
    lines = [ln for ln in raw
             if "packed-fp32-ops' is not a recognized feature" not in ln and "kernel-resource-usage" not in ln
             and not re.match(r"^\s*\d+ \|", ln) and not re.match(r"^\s*\|\s*\^", ln)
             and not ln.startswith("In file included from")]
    if proc.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return res


def build(jobs: int | None = None, verbose: bool = False, defines: list[str] | None = None,
          out: str | None = None) -> str:
    """Compile every source and link librowred.so (or `out`); returns the library path.

    `defines` are extra -D macros for the device sources (build variants)."""
    defines = defines or []
    tag = "_".join(d.replace("=", "") for d in defines)
    bdir = os.path.join(BUILD, tag) if tag else BUILD
    os.makedirs(bdir, exist_ok=True)
    lib = out or LIB
    cc = hipcc()
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *hip_flags(), "-Rpass-analysis=kernel-resource-usage",
                     *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(bdir, src.replace(".cpp", ".o"))
        objs.append(obj)
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
                     "-I/opt/rocm/include", "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)), 16)
    resources = {}
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for fut in [ex.submit(_run, c) for c in cmds]:
            resources.update(fut.result())
    with open(os.path.join(bdir, "resources.txt"), "w") as fh:
        for name in sorted(resources):
            r = resources[name]
            fh.write(f"{name} vgpr={r.get('vgpr')} agpr={r.get('agpr')} scratch={r.get('scratch')} "
                     f"lds={r.get('lds')} occupancy={r.get('occupancy')}\n")
    spilled = sorted(n for n, r in resources.items() if r.get("scratch", 0) > 0)
    if spilled:
        raise RuntimeError(f"{len(spilled)} kernel instance(s) use scratch memory (spills): "
                           + ", ".join(spilled[:5]))
    tmp = lib + f".tmp{os.getpid()}"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build librowred.so for gfx950")
    ap.add_argument("-D", "--define", action="append", default=[], help="extra device macro")
    ap.add_argument("-o", "--out", default=None, help="output library path")
    a = ap.parse_args()
    build(verbose=True, defines=a.define, out=a.out)

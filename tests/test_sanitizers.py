"""CPU sanitizer leg. The oracle (oracle/oracle.c) and the host code of the
library (argument validation and plan resolution in api.hip, the measurement
helpers' checks in measure.hip, the planner in plan.cpp) are built with
AddressSanitizer and UndefinedBehaviorSanitizer, and the CPU suites that
exercise them run against those builds in a child process (ORACLE_LIB and
ROWRED_LIB select them). The kernels' objects come from the regular build:
device code is not sanitized here, and its indexing is modelled on the host
in test_index_bounds.py. Two mistakes planted in a copy of oracle.c (a read
past an allocation, a signed overflow) check that the sanitizers are live."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "row_reduction_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "row_reduction_amd", "_build")
OUT = os.path.join(BUILD, "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LLVM_BIN = os.path.join(ROCM, "llvm", "bin")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

# clang (ROCm's LLVM) for everything, so one sanitizer runtime serves the
# process. On hipcc lines each sanitizer flag applies to the host side only.
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer", "-g", "-O1"]
SANITIZED_HIP = ("api.hip", "measure.hip")

SUITES = ["test_oracle.py", "test_abi.py", "test_index_bounds.py", "test_plan_model.py",
          "test_split_model.py", "test_concurrency.py", "test_zz_no_alloc.py"]


def asan_runtime() -> str:
    found = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.fail("clang's AddressSanitizer runtime is not installed under ROCm's LLVM")
    return found[0]


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]


def build_oracle(src: str, out: str) -> str:
    run([os.path.join(LLVM_BIN, "clang"), *SAN, "-ffp-contract=off", "-fPIC", "-shared", "-shared-libsan",
         src, "-o", out, "-lm"])
    return out


def build_library(out: str) -> str:
    """librowred with sanitized host code for the entry points and planner,
    linked with the regular build's kernel objects (built first if missing
    or older than their sources)."""
    from row_reduction_amd import build as rr_build
    kernel_objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in rr_build.HIP_SOURCES
                   if s not in SANITIZED_HIP]
    newest_src = max(os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*")) +
                     glob.glob(os.path.join(INCLUDE, "*")))
    if any(not os.path.exists(o) or os.path.getmtime(o) < newest_src for o in kernel_objs):
        rr_build.build()
    objs = []
    for src in SANITIZED_HIP:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        flags = [f for f in rr_build.hip_flags() if f != "-O3"]
        run([HIPCC, *flags, *HIP_HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    obj = os.path.join(OUT, "plan.o")
    run([os.path.join(LLVM_BIN, "clang++"), *SAN, "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
         f"-I{ROCM}/include", "-c", os.path.join(CSRC, "plan.cpp"), "-o", obj])
    objs.append(obj)
    run([os.path.join(LLVM_BIN, "clang++"), "-shared", *SAN[:1], "-shared-libsan", "-o", out, *objs,
         *kernel_objs, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    return out


def child_env(oracle_lib=None, rowred_lib=None) -> dict:
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan_runtime(), "ASAN_OPTIONS": "detect_leaks=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    if oracle_lib:
        env["ORACLE_LIB"] = oracle_lib
    if rowred_lib:
        env["ROWRED_LIB"] = rowred_lib
    return env


def test_cpu_suites_pass_on_sanitized_builds():
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(OUT, "liboracle_san.so"))
    rowred_lib = build_library(os.path.join(OUT, "librowred_san.so"))
    r = subprocess.run([sys.executable, "-m", "pytest", *[os.path.join(ROOT, "tests", f) for f in SUITES],
                        "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       capture_output=True, text=True, cwd=ROOT, env=child_env(oracle_lib, rowred_lib),
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-5000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]
    assert " passed" in r.stdout


PLANTED = [
    ("read past the end of an allocation", "out[r] = (float)sum_row(xr, cols);",
     "out[r] = (float)sum_row(xr, 4 * cols + 1);", "heap-buffer-overflow"),
    ("signed integer overflow", "out[r] = (float)sum_row(xr, cols);",
     "{ int k = 2147483647; k += (int)cols; out[r] = (float)sum_row(xr, cols + (k & 0)); }",
     "signed integer overflow"),
]


@pytest.mark.parametrize("name,old,new,report", PLANTED, ids=[p[0] for p in PLANTED])
def test_sanitizers_catch_a_planted_mistake(tmp_path, name, old, new, report):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1
    path = tmp_path / "oracle_planted.c"
    path.write_text(src.replace(old, new))
    lib = build_oracle(str(path), str(tmp_path / "liboracle_planted.so"))
    code = ("import sys, numpy as np; sys.path.insert(0, sys.argv[1]); import oracle; "
            "print(oracle.row_sum(np.ones((3, 5), np.float32)))")
    r = subprocess.run([sys.executable, "-c", code, ROOT], capture_output=True, text=True,
                       env=child_env(oracle_lib=lib), timeout=120)
    assert r.returncode != 0 and report in r.stderr, r.stdout[-2000:] + r.stderr[-2000:]

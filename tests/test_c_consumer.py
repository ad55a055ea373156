"""The C ABI from C (host only): a C99 program that includes only
include/rowred.h compiles warning-free with gcc, links against
librowred.so, and gets the documented results from the host-side calls."""
import os
import subprocess

from row_reduction_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_consumer_builds_links_and_runs(tmp_path):
    lib = _capi.LIB_PATH
    exe = tmp_path / "consumer"
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c_consumer", "consumer.c"),
                           "-o", str(exe), "-L", os.path.dirname(lib), "-lrowred",
                           "-Wl,-rpath," + os.path.dirname(lib)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"

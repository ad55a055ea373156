"""bench.py's command line on the CPU: it measures one GPU only, so a request
for more exits non-zero with a message saying so before touching a device,
and --help lists the documented options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode != 0
    msg = r.stdout + r.stderr
    assert "one GPU" in msg and "--gpus 2" in msg, msg


def test_help_lists_the_options():
    r = run("--help")
    assert r.returncode == 0, r.stderr
    for opt in ("--gpus", "--steps", "--warmup", "--no-shapes", "--no-cpu", "--detail"):
        assert opt in r.stdout, opt

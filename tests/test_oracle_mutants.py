"""The oracle's pins catch plausible mistakes (CPU only). Each case plants
one mistake in a copy of oracle/oracle.c (a dropped term, a wrong divisor, a
wrong sign or index, swapped operands, a rounding rule changed), builds it,
and runs the pins of tests/test_oracle.py for the function it touches against
that build in a fresh process (ORACLE_LIB): at least one pin must fail. The
unmodified source, built the same way, must pass them all."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

SOFTMAX_ROW = """    double z = 0.0;
    for (int64_t c = 0; c < cols; ++c) z += exp(x[c] - m);
    for (int64_t c = 0; c < cols; ++c) y[c] = exp(x[c] - m) / z;"""

# (name, text in oracle.c, replacement, pins to run: a pytest -k expression)
MUTANTS = [
    ("rmsnorm mean over cols + 1", "double mean_sq = sum_sq / (double)cols;",
     "double mean_sq = sum_sq / (double)(cols + 1);", "rmsnorm"),
    ("rmsnorm eps outside the root", "double denom = sqrt(mean_sq + eps);",
     "double denom = sqrt(mean_sq) + eps;", "rmsnorm"),
    ("rmsnorm weight dropped", "y[c] = x[c] * w[c] / denom;", "y[c] = x[c] / denom;", "rmsnorm"),
    ("rmsnorm signed square", "sum_sq += x[c] * x[c];", "sum_sq += x[c] * fabs(x[c]);", "rmsnorm"),
    ("rmsnorm first column skipped", "for (int64_t c = 0; c < cols; ++c) sum_sq += x[c] * x[c];",
     "for (int64_t c = 1; c < cols; ++c) sum_sq += x[c] * x[c];", "rmsnorm"),
    ("row sum first column skipped", "for (int64_t c = 0; c < cols; ++c) s += x[c];\n    return s;",
     "for (int64_t c = 1; c < cols; ++c) s += x[c];\n    return s;", "row_sum"),
    ("row sum in float32", "double s = 0.0;\n    for (int64_t c = 0; c < cols; ++c) s += x[c];",
     "float s = 0.0f;\n    for (int64_t c = 0; c < cols; ++c) s += (float)x[c];", "row_sum"),
    ("softmax sum without the max", SOFTMAX_ROW, SOFTMAX_ROW.replace("z += exp(x[c] - m)", "z += exp(x[c])"),
     "softmax"),
    ("softmax not normalised", SOFTMAX_ROW, SOFTMAX_ROW.replace("/ z;", ";"), "softmax"),
    ("softmax max replaced by first value",
     "static void softmax_row(const double *x, double *y, int64_t cols) {\n    double m = x[0];\n"
     "    for (int64_t c = 1; c < cols; ++c)\n        if (x[c] > m) m = x[c];",
     "static void softmax_row(const double *x, double *y, int64_t cols) {\n    double m = x[0];", "softmax"),
    ("layernorm unbiased variance", "double var = ss / (double)cols;",
     "double var = ss / (double)(cols > 1 ? cols - 1 : 1);", "layernorm"),
    ("layernorm beta dropped", "/ denom * gamma[c] + beta[c];", "/ denom * gamma[c];", "layernorm"),
    ("layernorm gamma and beta swapped", "/ denom * gamma[c] + beta[c];", "/ denom * beta[c] + gamma[c];",
     "layernorm"),
    ("layernorm eps outside the root", "double denom = sqrt(var + eps);", "double denom = sqrt(var) + eps;",
     "layernorm"),
    ("residual dropped", "double sum = hr[c] + load_elem(residual, s, r * cols + c);",
     "double sum = hr[c];", "residual"),
    ("residual sum not rounded to float32", "hr[c] = s == F32 ? (double)(float)sum :",
     "hr[c] = s == F32 ? sum :", "residual"),
    ("cross-entropy max dropped", "return log(z) + m - x[t];", "return log(z) - x[t];", "cross_entropy"),
    ("cross-entropy max replaced by first value",
     "    double m = x[0];\n    for (int64_t c = 1; c < cols; ++c)\n        if (x[c] > m) m = x[c];\n"
     "    double z = 0.0;\n    for (int64_t c = 0; c < cols; ++c) z += exp(x[c] - m);\n    return",
     "    double m = x[0];\n    double z = 0.0;\n    for (int64_t c = 0; c < cols; ++c) z += exp(x[c] - m);\n"
     "    return", "cross_entropy"),
    ("cross-entropy target sign", "return log(z) + m - x[t];", "return log(z) + m + x[t];", "cross_entropy"),
    ("bf16 ties away from zero", "double r = nearbyint(ldexp(fabs(v), -q));",
     "double r = round(ldexp(fabs(v), -q));", "bf16_rounding"),
    ("bf16 seven-bit significand", "int q = e - 8;", "int q = e - 7;", "bf16"),
    ("ownership worker index", "*worker = (i / V) % W;", "*worker = (i / W) % V;",
     "ownership or page_plans"),
    ("slot bound ignores the partial pack", "return full * V + (rem < V ? rem : V);",
     "return full * V + rem;", "ownership or page_plans"),
    ("long-row rmsnorm divisor", "double denom = sqrt(sum_sq / (double)cols + (double)eps);",
     "double denom = sqrt(sum_sq / (double)(cols + 1) + (double)eps);", "sampled"),
]


def build(src_text, path):
    c = str(path) + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    so = str(path) + ".so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", "-o", so, c, "-lm"])
    return so


def run_pins(so, k=None):
    env = dict(os.environ, ORACLE_LIB=so)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-x", "-q",
           "-p", "no:cacheprovider"]
    if k:
        cmd += ["-k", k]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_pins_pass_on_the_unmodified_source(tmp_path):
    r = run_pins(build(open(SRC).read(), tmp_path / "clean"))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new,k", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, k):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the planted text must occur exactly once"
    r = run_pins(build(src.replace(old, new), tmp_path / "mutant"), k)
    assert r.returncode == 1, f"{name}: no pin failed (pytest exit {r.returncode})\n{r.stdout[-2000:]}"
    assert " failed" in r.stdout, r.stdout[-2000:]

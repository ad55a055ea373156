"""The analytic plan model (host only): the C++ planner's predictions equal
the Python reference formulas, its choice is the cheapest legal candidate of
the search grid, the frozen constants reproduce the fit of the committed
timings and rank those timings as documented, and every choice is legal."""
import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import _capi, plan_model as pm, plans
from row_reduction_amd._capi import RR_OK

OPS = list(_capi.OP_IDS)


@pytest.fixture(scope="module")
def cases():
    return pm.load()


@pytest.fixture(scope="module")
def theta():
    return pm.read_inc()


def to_plan(d):
    return rr.rr_plan(d["path"], d["block"], d["lanes"], d["block"] // d["lanes"], d["v"], d["slots"], d["cache"])


def test_cpp_model_equals_python_reference(cases, theta):
    worst = 0.0
    for c in cases[::3]:
        for key in c["t"]:
            d = pm.parse_key(key)
            got = rr.rr_model_time_us(c["op"], c["rows"], c["cols"], to_plan(d))
            want = pm.predict_us(pm.features(c["op"], c["rows"], c["cols"], d), theta)
            worst = max(worst, abs(got - want) / want)
    assert worst <= 1e-12


@pytest.mark.parametrize("op", OPS)
def test_cpp_model_equals_python_reference_on_long_rows(op, theta):
    """The same agreement on rows past the register budget, where the
    streaming plans' LDS-held columns count as kept: every legal streaming
    candidate of three long shapes, with at least one holding values in LDS
    for the operators that can."""
    held = 0
    for rows, cols in ((256, 50257), (2048, 128256), (300, 200000)):
        for p in plans.candidate_plans(op, rows, cols, caches=(2,)):
            d = pm.parse_key(plans.plan_key(p))
            if d["path"] != 2:
                continue
            bf = op.endswith("_bf16")
            held += pm.lds_slots(op[:-5] if bf else op, bf, d) > 0
            got = rr.rr_model_time_us(op, rows, cols, p)
            want = pm.predict_us(pm.features(op, rows, cols, d), theta)
            assert abs(got - want) <= 1e-12 * want, (op, rows, cols, plans.plan_key(p))
    holds_lds = op.split("_bf16")[0] in ("softmax", "layernorm", "residual_layernorm") or op == "rmsnorm_bf16"
    assert (held > 0) == holds_lds


def model_cache(op, rows, cols):
    e = 2 if op.endswith("_bf16") else 4
    k = 3 if op.startswith("residual") else 2
    return 2 if e * rows * cols * k >= (1 << 20) else 0


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("shape", [(1, 1), (1, 127), (7, 96), (300, 777), (5000, 2048), (33, 40000), (70000, 64)])
def test_model_choice_is_cheapest_candidate(op, shape):
    rows, cols = shape
    cache = model_cache(op, rows, cols)
    cands = plans.candidate_plans(op, rows, cols, caches=(cache,))
    times = [rr.rr_model_time_us(op, rows, cols, p) for p in cands]
    assert all(t > 0 for t in times)
    best = cands[int(np.argmin(times))]
    got = rr.rr_select_plan_from(op, rows, cols, "model")
    assert got.as_dict() == best.as_dict()
    assert rr.rr_check_plan(op, rows, cols, got) == RR_OK


def test_frozen_constants_reproduce_the_fit(cases, theta):
    refit = pm.fit(cases)
    assert np.allclose(refit, theta, rtol=1e-6, atol=1e-12)


def test_in_sample_ranking_quality(cases, theta):
    """Regret of the model's pick against the fastest measured plan, over the
    360 (operator, shape) cases of the committed timings."""
    rg = pm.regrets(cases, theta)
    assert len(rg) == 360
    assert rg.mean() < 0.03 and np.median(rg) < 0.015 and rg.max() < 0.30


def test_auto_uses_table_then_model():
    # A table shape keeps its measured winner.
    assert rr.rr_select_plan("rmsnorm", 16384, 8192).as_dict() == \
        rr.rr_select_plan_from("rmsnorm", 16384, 8192, "table").as_dict()
    # Elsewhere the model decides.
    for op, rows, cols in [("rmsnorm", 3000, 5120), ("softmax_bf16", 12, 50000), ("sum", 70000, 40)]:
        with pytest.raises(rr.RowRedError):
            rr.rr_select_plan_from(op, rows, cols, "table")
        assert rr.rr_select_plan(op, rows, cols).as_dict() == \
            rr.rr_select_plan_from(op, rows, cols, "model").as_dict()


def test_every_source_returns_legal_plans():
    rng = np.random.default_rng(7)
    for _ in range(300):
        op = OPS[rng.integers(len(OPS))]
        rows = int(2 ** rng.uniform(0, 17))
        cols = int(2 ** rng.uniform(0, 18)) + 1
        for src in ("auto", "model", "rule"):
            p = rr.rr_select_plan_from(op, rows, cols, src)
            assert rr.rr_check_plan(op, rows, cols, p) == RR_OK, (op, rows, cols, src, p.as_dict())


def test_model_time_rejects_illegal_and_split_plans():
    assert rr.rr_model_time_us("rmsnorm", 64, 4096, rr.rr_plan(1, 256, 256, 1, 3, 12)) == -1.0
    split = rr.rr_plan(3, 256, 256, 1, 4, 16, 2)
    assert rr.rr_check_plan("rmsnorm", 4, 1 << 20, split) == RR_OK
    assert rr.rr_model_time_us("rmsnorm", 4, 1 << 20, split) == -1.0
    assert rr.rr_model_time_us(99, 64, 4096, rr.rr_plan(1, 256, 256, 1, 4, 16)) == -1.0
    L = _capi.lib()
    assert L.rr_select_plan_from(0, 64, 4096, 9, rr.rr_plan()) == _capi.RR_ERR_INVALID_ARGUMENT


def test_model_prefers_physically_sensible_plans():
    """Sanity of the terms on shapes far from the timings: a huge tensor is
    bandwidth-bound (prediction near bytes / 8 TB/s), one tiny row is near the
    launch floor, and a wider pack is never predicted slower on a big
    contiguous float row than the 1-wide pack of the same layout."""
    p = rr.rr_select_plan_from("rmsnorm", 32768, 4096, "model")
    t = rr.rr_model_time_us("rmsnorm", 32768, 4096, p)
    nbytes = 32768 * 4096 * 4 * 2
    assert nbytes / 8e6 <= t <= 2.0 * nbytes / 8e6
    p1 = rr.rr_select_plan_from("rmsnorm", 1, 64, "model")
    assert rr.rr_model_time_us("rmsnorm", 1, 64, p1) < 3.0
    for lanes in (256, 512, 1024):
        w1 = rr.rr_plan(1, lanes, lanes, 1, 1, 8192 // lanes, 2)
        w4 = rr.rr_plan(1, lanes, lanes, 1, 4, 8192 // lanes, 2)
        if rr.rr_check_plan("rmsnorm", 16384, 8192, w1) == RR_OK and rr.rr_check_plan("rmsnorm", 16384, 8192, w4) == RR_OK:
            assert rr.rr_model_time_us("rmsnorm", 16384, 8192, w4) <= rr.rr_model_time_us("rmsnorm", 16384, 8192, w1)

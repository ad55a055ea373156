"""The split-row selector of the *_ws entry points (host only): the C++
choice equals the Python reference formulas on a dense set of shapes, every
split it picks is a legal plan with the slice the rule describes, the frozen
constants reproduce the fit of the committed timings, and on the committed
held-out timings its choices stay close to the fastest plan timed."""
import statistics

import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import _capi, split_model as sm
from row_reduction_amd._capi import RR_OK, RR_PATH_SPLIT

OPS = list(_capi.OP_IDS)


@pytest.fixture(scope="module")
def theta():
    return sm.read_inc()


def shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = [(1, 8192), (1, 16384), (255, 1 << 20), (256, 1 << 20), (3, 100003), (1, 2047), (1, 2048),
           (2, 1 << 25), (1, (1 << 25) + 8), (65, 1000), (7, 40000)]
    for _ in range(n):
        rows = int(round(2 ** rng.uniform(0, 8.5)))
        cols = int(round(2 ** rng.uniform(10, 24)))
        out.append((rows, cols))
    return out


@pytest.mark.parametrize("op", OPS)
def test_cpp_choice_equals_python_reference(op, theta):
    for rows, cols in shapes(11 + OPS.index(op), 400):
        want = sm.choose(theta, op, rows, cols)
        got = rr.rr_workspace_bytes(op, rows, cols)
        if want == "plain":
            assert got == 0, (op, rows, cols)
            continue
        block, slots = map(int, want[1:].split("-k"))
        slices = -(-cols // (block * slots))
        assert got == rows * slices * 16, (op, rows, cols, want)
        p = rr.rr_plan(RR_PATH_SPLIT, block, block, 1, 8 if op.endswith("_bf16") else 4, slots, 2)
        assert rr.rr_check_plan(op, rows, cols, p) == RR_OK
        assert rr.rr_workspace_bytes(op, rows, cols, p) == got


def test_slice_rule():
    """16-slot slices: the narrowest workgroup giving 2..128 slices per row
    and at most 8192 workgroups; 1024 x 32 only where none does."""
    def k16_ok(rows, cols, b):
        s = -(-cols // (b * 16))
        return 2 <= s <= 128 and rows * s <= 8192

    for rows, cols in shapes(5, 2000):
        sp = sm.slice_plan("rmsnorm", rows, cols)
        wide_ok = 2 <= -(-cols // (1024 * 32)) <= 1024
        if sp is None:
            assert rows >= 256 or (not any(k16_ok(rows, cols, b) for b in sm.BLOCKS) and not wide_ok)
            continue
        block, slots = sp
        if slots == 16:
            assert k16_ok(rows, cols, block)
            assert not any(k16_ok(rows, cols, b) for b in sm.BLOCKS if b < block)
        else:
            assert (block, slots) == (1024, 32) and wide_ok
            assert not any(k16_ok(rows, cols, b) for b in sm.BLOCKS)
    assert sm.slice_plan("softmax_bf16", 3, 100003) is None          # bfloat16 rows need cols % 8 == 0
    assert sm.slice_plan("rmsnorm", 0, 1 << 20) is None
    assert sm.slice_plan("rmsnorm", 256, 1 << 20) is None


def test_frozen_constants_reproduce_the_fit(theta):
    fitted = sm.fit(sm.load(sm.DATA))
    for op in sm.OPS:
        np.testing.assert_allclose(theta[op], fitted[op], rtol=1e-9, err_msg=op)


def test_heldout_regret(theta):
    """On shapes none of the fitted timings lists (non-power-of-two rows and
    columns), the selector's choice is within 1.3 % of the fastest timed plan
    on average and never 20 % slower, against 15.8 % average regret for the
    earlier fixed rule (split whenever rows < 256 and cols >= 8192)."""
    cases = sm.load(sm.HELDOUT)
    train = {(c["rows"], c["cols"]) for c in sm.load(sm.DATA)}
    assert not ({(c["rows"], c["cols"]) for c in cases} & train)
    model = sm.regrets(cases, lambda c: sm.choose(theta, c["op"], c["rows"], c["cols"]))
    old = sm.regrets(cases, sm.old_rule)
    assert statistics.mean(model) <= 0.013
    assert max(model) <= 0.20
    assert statistics.mean(old) >= 0.15
    assert {c["op"] for c in cases} == set(sm.OPS)

"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a library
routine computing the same textbook definition in float64 (torch CPU, scipy,
math.fsum), a closed form, an invariant of the mathematics, or the worked
ownership example printed in the LuisaCompute "Consecutive-worker reduction
layout checkpoint" page ("Implementation and semantics" section).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from row_reduction_amd import workloads

TINY_COLS = (1, 2, 3, 31, 33, 127, 128, 129, 257)


def ulp_close(a, b, n_ulp=1):
    """|a - b| <= n_ulp units in the last place of float32 b, elementwise."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    spacing = np.spacing(np.abs(b)).astype(np.float64)
    return np.all(np.abs(a.astype(np.float64) - b.astype(np.float64)) <= n_ulp * spacing)


def family(rows, cols, seed=7):
    return workloads.family_inputs(rows, cols, seed)


def t64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


# ---------------------------------------------------------------- library routines

@pytest.mark.parametrize("cols", TINY_COLS)
@pytest.mark.parametrize("rows", [1, 5])
def test_rmsnorm_matches_torch_rms_norm_f64(rows, cols):
    wl = workloads.rmsnorm_workload(rows, cols, seed=11 + cols)
    y = oracle.rmsnorm(wl.x, wl.w, wl.eps)
    ref = F.rms_norm(t64(wl.x), (cols,), weight=t64(wl.w), eps=float(np.float32(wl.eps)))
    assert ulp_close(y, ref.numpy().astype(np.float32))


def test_rmsnorm_outlier_shape_matches_torch():
    wl = workloads.config_workloads(3)[0]
    y = oracle.rmsnorm(wl.x, wl.w, wl.eps)
    ref = F.rms_norm(t64(wl.x), (wl.cols,), weight=t64(wl.w), eps=float(np.float32(wl.eps)))
    assert wl.meta["outliers"] == round(0.01 * 64 * 4096)
    assert ulp_close(y, ref.numpy().astype(np.float32))


@pytest.mark.parametrize("cols", TINY_COLS)
def test_softmax_matches_scipy(cols):
    x = family(5, cols)["x"]
    y = oracle.softmax(x)
    ref = scipy.special.softmax(x.astype(np.float64), axis=1).astype(np.float32)
    assert ulp_close(y, ref)


@pytest.mark.parametrize("cols", TINY_COLS)
def test_layernorm_matches_torch_layer_norm_f64(cols):
    d = family(5, cols)
    eps = workloads.LAYERNORM_EPS
    y = oracle.layernorm(d["x"], d["gamma"], d["beta"], eps)
    ref = F.layer_norm(t64(d["x"]), (cols,), t64(d["gamma"]), t64(d["beta"]),
                       eps=float(np.float32(eps)))
    # y = z*gamma + beta can cancel; compare against the f64 result's own scale.
    ref = ref.numpy()
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-12)


@pytest.mark.parametrize("cols", TINY_COLS)
def test_residual_layernorm_h_is_float32_sum_and_y_matches_torch(cols):
    d = family(5, cols)
    eps = workloads.LAYERNORM_EPS
    y, h = oracle.residual_layernorm(d["x"], d["residual"], d["gamma"], d["beta"], eps)
    h_ref = d["x"] + d["residual"]                    # numpy float32 add: one rounding
    assert np.array_equal(h.view(np.int32), h_ref.view(np.int32))
    ref = F.layer_norm(t64(h_ref), (cols,), t64(d["gamma"]), t64(d["beta"]),
                       eps=float(np.float32(eps))).numpy()
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-12)


@pytest.mark.parametrize("cols", TINY_COLS)
def test_cross_entropy_matches_torch_f64(cols):
    d = family(5, cols)
    loss = oracle.cross_entropy(d["x"], d["targets"])
    ref = F.cross_entropy(t64(d["x"]), torch.from_numpy(d["targets"].astype(np.int64)),
                          reduction="none").numpy()
    err = np.abs(loss.astype(np.float64) - ref)
    assert np.all(err <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-12)


@pytest.mark.parametrize("cols", TINY_COLS)
def test_row_sum_matches_fsum(cols):
    x = family(5, cols)["x"]
    out = oracle.row_sum(x)
    ref = np.array([math.fsum(map(float, row)) for row in x], np.float64)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-30)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("c", [0.75, -0.75, 3.0, 1e-3, -2.5])
@pytest.mark.parametrize("cols", [1, 33, 257])
def test_rmsnorm_constant_row_closed_form(c, cols):
    """Constant row c: y = sign(c) * w * |c| / sqrt(c^2 + eps)."""
    eps = np.float32(1e-6)
    x = np.full((2, cols), c, np.float32)
    w = np.linspace(0.5, 1.5, cols, dtype=np.float32)
    y = oracle.rmsnorm(x, w, eps)
    cf = float(np.float32(c))
    ref = np.array([math.copysign(1.0, cf) * float(wc) * abs(cf) / math.sqrt(cf * cf + float(eps))
                    for wc in w], np.float64).astype(np.float32)
    assert ulp_close(y, np.broadcast_to(ref, y.shape))


@pytest.mark.parametrize("cols", [1, 2, 31, 128, 257, 4103])
def test_softmax_constant_row_is_uniform(cols):
    y = oracle.softmax(np.full((3, cols), -1.25, np.float32))
    assert np.all(y == np.float32(1.0 / cols))


@pytest.mark.parametrize("cols", [2, 31, 257, 4103])
def test_masked_softmax_is_softmax_of_the_survivors(cols):
    """-inf entries (masked positions): probability exactly 0, and the other
    entries are the softmax of the unmasked ones alone (scipy on the subset);
    cross-entropy is the subset's, +inf for a masked target; a fully masked
    row is NaN."""
    rng = np.random.default_rng(cols)
    x = family(3, cols)["x"]
    mask = rng.random((3, cols)) < 0.4
    mask[:, 0] = False
    mask[2, :] = True
    x[mask] = -np.inf
    y = oracle.softmax(x)
    for r in range(2):
        keep = ~mask[r]
        assert np.all(y[r, mask[r]] == 0.0)
        ref = scipy.special.softmax(x[r, keep].astype(np.float64)).astype(np.float32)
        assert ulp_close(y[r, keep], ref)
    assert np.isnan(y[2]).all()
    t = np.array([0, int(np.flatnonzero(mask[1])[0]) if mask[1].any() else 0, 0], np.int32)
    loss = oracle.cross_entropy(x, t)
    ref0 = -math.log(scipy.special.softmax(x[0, ~mask[0]].astype(np.float64))[0])
    assert ulp_close(loss[:1], np.array([ref0], np.float32))
    if mask[1].any():
        assert loss[1] == np.inf
    assert np.isnan(loss[2])


@pytest.mark.parametrize("cols", [1, 2, 31, 128, 257, 4103])
def test_cross_entropy_constant_row_is_log_cols(cols):
    x = np.full((3, cols), 0.5, np.float32)
    loss = oracle.cross_entropy(x, np.array([0, cols - 1, cols // 2], np.int32))
    assert ulp_close(loss, np.full(3, math.log(cols), np.float32))


@pytest.mark.parametrize("cols", [1, 2, 31, 128, 257])
def test_layernorm_constant_row_gives_beta(cols):
    d = family(2, cols)
    x = np.full((2, cols), 0.75, np.float32)
    y = oracle.layernorm(x, d["gamma"], d["beta"], 1e-5)
    assert np.array_equal(y, np.broadcast_to(d["beta"], y.shape))


@pytest.mark.parametrize("cols", [1, 31, 257, 4096])
def test_row_sum_small_integers_exact(cols):
    x = np.full((2, cols), 3.0, np.float32)
    x[1] = np.arange(cols) % 7 - 3
    out = oracle.row_sum(x)
    assert out[0] == 3.0 * cols and out[1] == float(np.sum(np.arange(cols) % 7 - 3))


def test_cols_one_special_cases():
    x = np.array([[2.0], [-0.5], [0.0]], np.float32)
    assert np.all(oracle.softmax(x) == 1.0)
    assert np.all(oracle.cross_entropy(x, np.zeros(3, np.int32)) == 0.0)
    assert np.array_equal(oracle.layernorm(x, [2.0], [0.25], 1e-5), np.full((3, 1), 0.25, np.float32))
    assert np.array_equal(oracle.row_sum(x), x[:, 0])


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("k", [-3, 1, 5])
def test_rmsnorm_power_of_two_scale_invariance_bitwise(k):
    wl = workloads.rmsnorm_workload(5, 257, seed=3)
    y1 = oracle.rmsnorm(wl.x, wl.w, 0.0)
    y2 = oracle.rmsnorm(wl.x * np.float32(2.0 ** k), wl.w, 0.0)
    assert np.array_equal(y1.view(np.int32), y2.view(np.int32))


@pytest.mark.parametrize("alpha", [0.3, 7.0, 1234.5])
def test_rmsnorm_positive_scale_invariance(alpha):
    wl = workloads.rmsnorm_workload(5, 129, seed=4)
    y1 = oracle.rmsnorm(wl.x, wl.w, 0.0)
    y2 = oracle.rmsnorm((wl.x.astype(np.float64) * alpha).astype(np.float32), wl.w, 0.0)
    assert np.all(np.abs(y1 - y2) <= 1e-5 + 1e-5 * np.abs(y1))


def test_rmsnorm_unit_magnitude_identity():
    """x in {-1, +1}, w = 1, eps = 0 gives y = x exactly (mean square is 1)."""
    rng = np.random.default_rng(0)
    x = np.where(rng.random((4, 257)) < 0.5, -1.0, 1.0).astype(np.float32)
    y = oracle.rmsnorm(x, np.ones(257, np.float32), 0.0)
    assert np.array_equal(y, x)


def test_rmsnorm_signed_zero():
    x = np.array([[-0.0, 1.0, 0.0, -2.0]], np.float32)
    y = oracle.rmsnorm(x, np.ones(4, np.float32), 1e-6)
    assert np.signbit(y[0, 0]) and not np.signbit(y[0, 2])


@pytest.mark.parametrize("cols", [1, 31, 127, 257, 4103])
def test_softmax_rows_sum_to_one(cols):
    y = oracle.softmax(family(5, cols)["x"])
    assert np.all(y >= 0) and np.all(y <= 1)
    assert np.all(np.abs(y.astype(np.float64).sum(axis=1) - 1.0) <= 1e-5)


def test_softmax_and_cross_entropy_large_logits_do_not_overflow():
    """Logits 800 apart: exp of the raw values would overflow even float64;
    with the row maximum subtracted first the results are exact: the large
    entry takes all the mass (the other's e^-800 is below float32's range),
    and the loss is 800 at the small entry, 0 at the large one."""
    x = np.array([[0.0, 800.0], [800.0, 0.0], [-800.0, 0.0], [0.0, -800.0]], np.float32)
    y = oracle.softmax(x)
    assert np.array_equal(y, np.array([[0, 1], [1, 0], [0, 1], [1, 0]], np.float32))
    loss = oracle.cross_entropy(x, np.array([0, 0, 1, 1], np.int32))
    assert np.array_equal(loss, np.array([800, 0, 0, 800], np.float32))


def test_softmax_shift_invariance_bitwise():
    rng = np.random.default_rng(1)
    x = (rng.integers(-512, 512, size=(4, 129)) / 64.0).astype(np.float32)  # exact in f32
    assert np.array_equal(oracle.softmax(x), oracle.softmax(x + np.float32(4.0)))


def test_cross_entropy_is_negative_log_softmax_at_target():
    d = family(5, 257)
    loss = oracle.cross_entropy(d["x"], d["targets"])
    p = oracle.softmax(d["x"])[np.arange(5), d["targets"]].astype(np.float64)
    assert np.all(loss >= 0)
    assert np.all(np.abs(loss + np.log(p)) <= 1e-5 + 1e-5 * np.abs(loss))


def test_cross_entropy_target_out_of_range_is_nan():
    x = family(3, 33)["x"]
    loss = oracle.cross_entropy(x, np.array([-1, 33, 0], np.int32))
    assert np.isnan(loss[0]) and np.isnan(loss[1]) and np.isfinite(loss[2])


def test_residual_layernorm_zero_residual_equals_layernorm():
    d = family(5, 257)
    y, h = oracle.residual_layernorm(d["x"], np.zeros_like(d["x"]), d["gamma"], d["beta"], 1e-5)
    assert np.array_equal(h, d["x"])
    assert np.array_equal(y, oracle.layernorm(d["x"], d["gamma"], d["beta"], 1e-5))


def test_layernorm_unit_affine_moments():
    d = family(5, 4096)
    x = d["x"].astype(np.float64)
    eps = 1e-5
    y = oracle.layernorm(d["x"], np.ones(4096, np.float32), np.zeros(4096, np.float32), eps)
    var = x.var(axis=1)
    yd = y.astype(np.float64)
    assert np.all(np.abs(yd.mean(axis=1)) <= 1e-6)
    assert np.allclose((yd ** 2).mean(axis=1), var / (var + np.float32(eps)), rtol=1e-6, atol=0)


def test_rejects_bad_shape():
    with pytest.raises(ValueError):
        oracle.rmsnorm(np.zeros((2, 0), np.float32), np.zeros(0, np.float32), 1e-6)


# ---------------------------------------------------------------- ownership map

def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_ownership_matches_printed_w4_v2_example():
    W, V = 4, 2
    rows = _golden_rows("ownership_w4_v2.txt")
    assert len(rows) == 8
    for chunk, worker, e0, e1 in rows:
        for element, i in enumerate((e0, e1)):
            slot = chunk * V + element
            assert oracle.logical_index(worker, slot, W, V) == i
            assert oracle.owner(i, W, V) == (worker, slot)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8, 32, 64, 96, 256])
@pytest.mark.parametrize("V", [1, 2, 4, 8])
def test_ownership_bijection_and_slot_bound_brute_force(W, V):
    for N in list(range(0, 70)) + [127, 128, 129, 257, 1000, 4103]:
        seen = set()
        per_worker = {}
        for i in range(N):
            wk, sl = oracle.owner(i, W, V)
            assert 0 <= wk < W
            assert (wk, sl) not in seen
            seen.add((wk, sl))
            assert oracle.logical_index(wk, sl, W, V) == i
            per_worker[wk] = per_worker.get(wk, 0) + 1
        brute = max(per_worker.values()) if per_worker else 0
        assert oracle.slot_bound(N, W, V) == brute, (N, W, V)


def test_page_plans_slot_counts_by_enumeration():
    """The page's chosen worker/V pairs: the bound equals the enumerated maximum."""
    for rows, cols, W, V in _golden_rows("page_plans.txt"):
        counts = {}
        for i in range(cols):
            wk = (i // V) % W            # owner by counting runs of V across W workers
            counts[wk] = counts.get(wk, 0) + 1
        assert oracle.slot_bound(cols, W, V) == max(counts.values())


# ---------------------------------------------------------------- bfloat16 storage

def torch_bf16_bits(a32):
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_ulp(b):
    """Unit in the last place of bfloat16 values (as float64)."""
    v = np.abs(oracle.bf16_to_float(b).astype(np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -133)))
    return np.maximum(2.0 ** (e - 7), 2.0 ** -133)


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(5)
    vals = [rng.normal(0, 1, 2000), rng.normal(0, 1, 2000) * 10.0 ** rng.integers(-40, 38, 2000),
            [0.0, -0.0, 1.0, -1.0, 3.0e38, 3.3895313e38, -3.3895313e38, 1e-40, -1e-40, 1.2e-38]]
    x = np.concatenate([np.asarray(v, np.float64) for v in vals]).astype(np.float32)
    # Exact ties: a bfloat16 value plus half its quantum (low half 0x8000).
    base = torch_bf16_bits(rng.normal(0, 1, 500).astype(np.float32)).astype(np.uint32)
    ties = ((base << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, torch_bf16_bits(x))


def test_bf16_rounding_directed_cases():
    one = 1.0
    q = 2.0 ** -7                      # quantum of bfloat16 in [1, 2)
    assert oracle.bf16_from_double(one + q / 2) == 0x3f80          # tie -> even (1.0)
    assert oracle.bf16_from_double(one + q / 2 + 2.0 ** -40) == 0x3f81  # just above the tie
    assert oracle.bf16_from_double(one + 1.5 * q) == 0x3f82        # tie -> even (1 + 2q)
    assert oracle.bf16_from_double(one + 1.5 * q - 2.0 ** -40) == 0x3f81
    assert oracle.bf16_from_double(2.0 - q / 4) == 0x4000          # rounds up across the binade
    assert oracle.bf16_from_double(float("inf")) == 0x7f80
    assert oracle.bf16_from_double(3.5e38) == 0x7f80               # overflow -> inf
    assert oracle.bf16_from_double(-3.5e38) == 0xff80
    assert oracle.bf16_from_double(2.0 ** -133) == 0x0001          # smallest subnormal
    assert oracle.bf16_from_double(2.0 ** -135) == 0x0000          # below half of it
    assert oracle.bf16_from_double(float("nan")) & 0x7f80 == 0x7f80


@pytest.mark.parametrize("cols", [1, 33, 257, 4096])
def test_bf16_row_sum_and_cross_entropy_equal_f32_oracle_on_widened_inputs(cols):
    d = workloads.family_inputs_bf16(5, cols, seed=12)
    x32 = oracle.bf16_to_float(d["x"])
    assert np.array_equal(oracle.row_sum_bf16(d["x"]), oracle.row_sum(x32))
    assert np.array_equal(oracle.cross_entropy_bf16(d["x"], d["targets"]),
                          oracle.cross_entropy(x32, d["targets"]))


def _within_bf16_ulp(got_bits, ref64):
    g = oracle.bf16_to_float(got_bits).astype(np.float64)
    ref_bits = torch_bf16_bits(ref64.astype(np.float32))
    ok = np.abs(g - ref64) <= bf16_ulp(ref_bits)
    exact = np.mean(got_bits == ref_bits)
    return bool(np.all(ok)), exact


@pytest.mark.parametrize("cols", [1, 31, 257, 4096])
def test_bf16_rmsnorm_softmax_layernorm_match_library_routines(cols):
    d = workloads.family_inputs_bf16(5, cols, seed=13)
    x64 = t64(oracle.bf16_to_float(d["x"]))
    g64 = t64(oracle.bf16_to_float(d["gamma"]))
    b64 = t64(oracle.bf16_to_float(d["beta"]))
    eps = float(np.float32(1e-5))
    cases = [
        (oracle.rmsnorm_bf16(d["x"], d["gamma"], 1e-5), F.rms_norm(x64, (cols,), weight=g64, eps=eps)),
        (oracle.softmax_bf16(d["x"]), torch.softmax(x64, dim=1)),
        (oracle.layernorm_bf16(d["x"], d["gamma"], d["beta"], 1e-5),
         F.layer_norm(x64, (cols,), g64, b64, eps=eps)),
    ]
    for got, ref in cases:
        ok, exact = _within_bf16_ulp(got, ref.numpy())
        assert ok and exact > 0.99


def test_bf16_residual_layernorm_h_is_one_rounding_of_the_sum():
    d = workloads.family_inputs_bf16(5, 257, seed=14)
    y, h = oracle.residual_layernorm_bf16(d["x"], d["residual"], d["gamma"], d["beta"], 1e-5)
    hs = torch.from_numpy(oracle.bf16_to_float(d["x"])).double() + \
        torch.from_numpy(oracle.bf16_to_float(d["residual"])).double()
    assert np.array_equal(h, torch_bf16_bits(hs.float().numpy()))
    ref = F.layer_norm(torch.from_numpy(oracle.bf16_to_float(h)).double(), (257,),
                       t64(oracle.bf16_to_float(d["gamma"])), t64(oracle.bf16_to_float(d["beta"])),
                       eps=float(np.float32(1e-5)))
    ok, exact = _within_bf16_ulp(y, ref.numpy())
    assert ok and exact > 0.99


def test_bf16_rmsnorm_constant_row_closed_form():
    c = 0.75
    w = workloads.as_bf16_bits(np.linspace(0.5, 1.5, 64, dtype=np.float32))
    x = workloads.as_bf16_bits(np.full((2, 64), c, np.float32))
    y = oracle.rmsnorm_bf16(x, w, 1e-6)
    wf = oracle.bf16_to_float(w).astype(np.float64)
    ref = wf * c / math.sqrt(c * c + float(np.float32(1e-6)))
    ok, exact = _within_bf16_ulp(y[0], ref)
    assert ok and np.array_equal(y[0], y[1])


@pytest.mark.parametrize("cols", [1, 2, 31, 257, 4103, 100003])
def test_sampled_long_row_forms_equal_the_full_row_oracle(cols):
    """The one-row forms for very long rows (statistic over the whole row,
    outputs at chosen columns, no float64 copy of the row) give exactly the
    full-row oracle's values: same definitions, same accumulation order."""
    rng = np.random.default_rng(cols)
    x = rng.standard_normal(cols).astype(np.float32)
    w = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    idx = np.unique(np.concatenate([[0, cols - 1], rng.integers(0, cols, 64)]))
    assert np.array_equal(oracle.rmsnorm_sampled(x, w, 1e-6, idx), oracle.rmsnorm(x[None], w, 1e-6)[0][idx])
    assert np.array_equal(oracle.softmax_sampled(x, idx), oracle.softmax(x[None])[0][idx])
    assert oracle.row_sum_long(x) == oracle.row_sum(x[None])[0]


def test_sampled_long_row_forms_match_numpy_f64():
    """Against numpy's float64 (pairwise) sums on a 3M-column row: within one
    float32 ulp of the rounded results."""
    rng = np.random.default_rng(77)
    cols = 3_000_017
    x = rng.standard_normal(cols).astype(np.float32)
    w = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    idx = rng.integers(0, cols, 256)
    x64 = x.astype(np.float64)
    ref = (x64[idx] * w[idx] / np.sqrt(np.sum(x64 * x64) / cols + np.float64(np.float32(1e-6)))).astype(np.float32)
    assert ulp_close(oracle.rmsnorm_sampled(x, w, 1e-6, idx), ref)
    e = np.exp(x64 - x64.max())
    assert ulp_close(oracle.softmax_sampled(x, idx), (e[idx] / e.sum()).astype(np.float32))
    assert ulp_close(np.array([oracle.row_sum_long(x)]), np.array([math.fsum(x64)], np.float32))


@pytest.mark.parametrize("cols", [1, 2, 3, 31, 33, 127, 128, 129, 257])
def test_every_operator_matches_pure_python_brute_force(cols):
    """Every operator against tests/brute.py (pure Python: math.fsum sums,
    float64 sqrt/exp/log, one rounding) on tiny inputs, within one float32
    ulp."""
    import brute
    d = family(5, cols, seed=cols)
    x, g, b, r, t = d["x"], d["gamma"], d["beta"], d["residual"], d["targets"]
    w = g
    assert ulp_close(oracle.rmsnorm(x, w, 1e-6), brute.rmsnorm(x, w, 1e-6))
    assert ulp_close(oracle.row_sum(x), brute.row_sum(x))
    assert ulp_close(oracle.softmax(x), brute.softmax(x))
    assert ulp_close(oracle.layernorm(x, g, b, 1e-5), brute.layernorm(x, g, b, 1e-5))
    y, h = oracle.residual_layernorm(x, r, g, b, 1e-5)
    yb, hb = brute.residual_layernorm(x, r, g, b, 1e-5)
    assert np.array_equal(h, hb)
    assert ulp_close(y, yb)
    assert ulp_close(oracle.cross_entropy(x, t), brute.cross_entropy(x, t))

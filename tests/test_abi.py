"""C-ABI library: loads, exports what include/rowred.h declares, validates
arguments and plans on the host (no GPU, no kernel launch)."""
import ctypes
import os
import re

import pytest

import oracle
from row_reduction_amd import _capi, workloads
from row_reduction_amd._capi import (RR_ERR_INVALID_ARGUMENT, RR_ERR_UNSUPPORTED, RR_OK,
                                     RR_PATH_LOOP, RR_PATH_PACKED, RR_PATH_ROW, RR_PATH_SPLIT,
                                     rr_plan)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rowred.h")

# Non-null, dword-aligned stand-ins: every call below is rejected on the host
# before any device work, so these are never dereferenced.
P = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10002)
NULL = None


@pytest.fixture(scope="module")
def L():
    return _capi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int64_t|int|double|const\s+char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    assert set(names) == set(_capi.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert _capi.status_string(RR_OK) == "RR_OK"
    assert _capi.status_string(RR_ERR_INVALID_ARGUMENT) == "RR_ERR_INVALID_ARGUMENT"
    assert _capi.status_string(RR_ERR_UNSUPPORTED) == "RR_ERR_UNSUPPORTED"
    assert _capi.status_string(3) == "RR_ERR_LAUNCH"
    assert _capi.status_string(99) == "RR_UNKNOWN_STATUS"


# ---------------------------------------------------------------- argument errors

def call(L, op, x=P, rows=4, cols=8, eps=1e-6, plan=None, **kw):
    """Invoke one entry point with stand-in pointers, overriding some."""
    if op.endswith("_bf16"):
        return call_bf16(L, op[:-5], x, rows, cols, eps, plan, **kw)
    if op == "rmsnorm":
        return L.rmsnorm_f32_ex(x, kw.get("w", P), kw.get("y", P), rows, cols, eps, plan, None)
    if op == "sum":
        return L.row_sum_f32_ex(x, kw.get("out", P), rows, cols, plan, None)
    if op == "softmax":
        return L.softmax_f32_ex(x, kw.get("y", P), rows, cols, plan, None)
    if op == "layernorm":
        return L.layernorm_f32_ex(x, kw.get("gamma", P), kw.get("beta", P), kw.get("y", P), rows,
                                  cols, eps, plan, None)
    if op == "residual_layernorm":
        return L.residual_layernorm_f32_ex(x, kw.get("residual", P), kw.get("gamma", P),
                                           kw.get("beta", P), kw.get("y", P), kw.get("h", None),
                                           rows, cols, eps, plan, None)
    if op == "cross_entropy":
        return L.cross_entropy_f32_ex(x, kw.get("targets", P), kw.get("loss", P), rows, cols, plan,
                                      None)
    raise ValueError(op)


def call_bf16(L, op, x, rows, cols, eps, plan, **kw):
    if op == "rmsnorm":
        return L.rmsnorm_bf16_ex(x, kw.get("w", P), kw.get("y", P), rows, cols, eps, plan, None)
    if op == "sum":
        return L.row_sum_bf16_ex(x, kw.get("out", P), rows, cols, plan, None)
    if op == "softmax":
        return L.softmax_bf16_ex(x, kw.get("y", P), rows, cols, plan, None)
    if op == "layernorm":
        return L.layernorm_bf16_ex(x, kw.get("gamma", P), kw.get("beta", P), kw.get("y", P), rows,
                                   cols, eps, plan, None)
    if op == "residual_layernorm":
        return L.residual_layernorm_bf16_ex(x, kw.get("residual", P), kw.get("gamma", P),
                                            kw.get("beta", P), kw.get("y", P), kw.get("h", None),
                                            rows, cols, eps, plan, None)
    if op == "cross_entropy":
        return L.cross_entropy_bf16_ex(x, kw.get("targets", P), kw.get("loss", P), rows, cols, plan,
                                       None)
    raise ValueError(op)


OPS = list(_capi.OP_IDS)
MISALIGNED_BF16 = ctypes.c_void_p(0x10001)
FLOAT_OUTS = {"sum": "out", "cross_entropy": "loss"}


@pytest.mark.parametrize("op", OPS)
def test_rows_zero_is_ok_without_launch(L, op):
    assert call(L, op, rows=0) == RR_OK
    # Even with null pointers: nothing is touched.
    assert call(L, op, x=NULL, rows=0) == RR_OK


@pytest.mark.parametrize("op", OPS)
def test_bad_shapes(L, op):
    assert call(L, op, rows=-1) == RR_ERR_INVALID_ARGUMENT
    assert call(L, op, cols=0) == RR_ERR_INVALID_ARGUMENT
    assert call(L, op, cols=-5) == RR_ERR_INVALID_ARGUMENT
    assert call(L, op, cols=1 << 31) == RR_ERR_UNSUPPORTED
    assert call(L, op, cols=_capi.RR_MAX_COLS + 1) == RR_ERR_UNSUPPORTED
    assert call(L, op, rows=0, cols=_capi.RR_MAX_COLS) == RR_OK


@pytest.mark.parametrize("op", OPS)
def test_null_and_misaligned_pointers(L, op):
    bf16 = op.endswith("_bf16")
    base = op[:-5] if bf16 else op
    bad = MISALIGNED_BF16 if bf16 else MISALIGNED
    assert call(L, op, x=NULL) == RR_ERR_INVALID_ARGUMENT
    assert call(L, op, x=bad) == RR_ERR_INVALID_ARGUMENT
    out_kw = {"rmsnorm": "y", "sum": "out", "softmax": "y", "layernorm": "y",
              "residual_layernorm": "y", "cross_entropy": "loss"}[base]
    assert call(L, op, **{out_kw: NULL}) == RR_ERR_INVALID_ARGUMENT
    # Float per-row outputs need 4-byte alignment even for bfloat16 inputs.
    out_bad = MISALIGNED if (not bf16 or base in FLOAT_OUTS) else bad
    assert call(L, op, **{out_kw: out_bad}) == RR_ERR_INVALID_ARGUMENT


def test_operator_specific_pointers(L):
    assert call(L, "rmsnorm", w=NULL) == RR_ERR_INVALID_ARGUMENT
    assert call(L, "layernorm", gamma=NULL) == RR_ERR_INVALID_ARGUMENT
    assert call(L, "layernorm", beta=MISALIGNED) == RR_ERR_INVALID_ARGUMENT
    assert call(L, "residual_layernorm", residual=NULL) == RR_ERR_INVALID_ARGUMENT
    assert call(L, "residual_layernorm", h=MISALIGNED) == RR_ERR_INVALID_ARGUMENT
    assert call(L, "cross_entropy", targets=NULL) == RR_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("op", ["rmsnorm", "layernorm", "residual_layernorm"])
@pytest.mark.parametrize("eps", [-1e-6, float("nan"), float("inf")])
def test_bad_eps(L, op, eps):
    assert call(L, op, eps=eps) == RR_ERR_INVALID_ARGUMENT


# ---------------------------------------------------------------- plans

def plan(path, block, lanes, v, slots):
    return rr_plan(path, block, lanes, block // lanes, v, slots)


ILLEGAL = [
    plan(RR_PATH_ROW, 256, 256, 3, 12),        # V = 3
    plan(RR_PATH_ROW, 256, 96, 4, 16),         # lanes not a power of two
    plan(RR_PATH_ROW, 2048, 1024, 4, 16),      # block above 1024
    plan(RR_PATH_ROW, 32, 32, 4, 16),          # block below one wavefront
    plan(RR_PATH_ROW, 256, 512, 4, 16),        # lanes > block
    plan(RR_PATH_ROW, 256, 256, 4, 64),        # 16 chunks: over the register budget
    plan(RR_PATH_ROW, 256, 256, 4, 12),        # 3 chunks: not a power of two
    plan(RR_PATH_ROW, 256, 64, 4, 4),          # too few slots for 4096 columns
    plan(RR_PATH_ROW, 256, 32, 4, 32),         # ROW needs >= 64 lanes
    plan(RR_PATH_PACKED, 256, 64, 4, 16),      # PACKED needs < 64 lanes
    plan(RR_PATH_LOOP, 256, 128, 4, 0),        # LOOP: one row per group
    plan(RR_PATH_LOOP, 256, 256, 4, 16),       # LOOP keeps 0 or 32 slots
    plan(RR_PATH_LOOP, 256, 256, 2, 32),       # LOOP keeps slots only at V >= 4
    rr_plan(RR_PATH_ROW, 256, 128, 1, 4, 16),  # rows_per_group inconsistent
    rr_plan(7, 256, 256, 1, 4, 16),            # unknown path
    rr_plan(RR_PATH_ROW, 256, 256, 1, 4, 16, 3),   # unknown cache policy
    rr_plan(RR_PATH_ROW, 256, 256, 1, 4, 16, -1),  # unknown cache policy
]


@pytest.mark.parametrize("bad", ILLEGAL, ids=lambda p: str(p.as_dict()))
def test_illegal_plans_fail_closed(L, bad):
    assert L.rr_check_plan(0, 64, 4096, bad) == RR_ERR_UNSUPPORTED
    # The entry points refuse them before launching anything.
    for op in OPS:
        assert call(L, op, rows=64, cols=4096, plan=bad) == RR_ERR_UNSUPPORTED


def test_bf16_pack_width_rules(L):
    rms16 = _capi.OP_IDS["rmsnorm_bf16"]
    # V = 8 exists only for bfloat16 rows.
    assert L.rr_check_plan(0, 64, 4096, plan(RR_PATH_ROW, 256, 256, 8, 16)) == RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(rms16, 64, 4096, plan(RR_PATH_ROW, 256, 256, 8, 16)) == RR_OK
    # At most 32 live values per lane: 8 packs of 8 is over.
    assert L.rr_check_plan(rms16, 64, 4096, plan(RR_PATH_ROW, 64, 64, 8, 64)) == RR_ERR_UNSUPPORTED
    # V > 1 needs cols % V == 0 (naturally aligned packs).
    assert L.rr_check_plan(rms16, 5, 257, plan(RR_PATH_ROW, 64, 64, 4, 8)) == RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(rms16, 5, 257, plan(RR_PATH_ROW, 64, 64, 1, 8)) == RR_OK
    assert L.rr_check_plan(rms16, 5, 258, plan(RR_PATH_ROW, 64, 64, 2, 8)) == RR_OK
    p = rr_plan()
    assert L.rr_select_plan(rms16, 5, 257, p) == RR_OK and p.v == 1
    assert L.rr_select_plan(rms16, 1024, 4096, p) == RR_OK and 4096 % p.v == 0


def test_bf16_explicit_plan_needs_pointer_alignment(L):
    """Pointers only 2-byte aligned cannot take 4-byte packs: refused, not remapped."""
    p2 = ctypes.c_void_p(0x10002)
    wide = plan(RR_PATH_ROW, 64, 64, 2, 2)
    assert L.rmsnorm_bf16_ex(p2, P, P, 4, 128, 1e-6, wide, None) == RR_ERR_UNSUPPORTED
    assert L.softmax_bf16_ex(P, p2, 4, 128, wide, None) == RR_ERR_UNSUPPORTED


def test_streaming_kept_slots_only_for_two_pass_operators(L):
    kept = plan(RR_PATH_LOOP, 1024, 1024, 4, 32)
    for op in ("rmsnorm", "softmax", "layernorm", "residual_layernorm"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 100000, kept) == RR_OK
    for op in ("sum", "cross_entropy"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 100000, kept) == RR_ERR_UNSUPPORTED
    wide = plan(RR_PATH_LOOP, 1024, 1024, 4, 64)
    for op in ("rmsnorm", "softmax", "rmsnorm_bf16", "softmax_bf16"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 100000, wide) == RR_OK
    for op in ("layernorm", "residual_layernorm", "sum", "cross_entropy"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 100000, wide) == RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(0, 3, 100000, plan(RR_PATH_LOOP, 256, 256, 4, 64)) == RR_ERR_UNSUPPORTED
    kept8 = plan(RR_PATH_LOOP, 1024, 1024, 8, 32)
    assert L.rr_check_plan(_capi.OP_IDS["softmax_bf16"], 3, 100000, kept8) == RR_OK
    assert L.rr_check_plan(_capi.OP_IDS["cross_entropy_bf16"], 3, 100000, kept8) == RR_ERR_UNSUPPORTED
    vocab = plan(RR_PATH_LOOP, 1024, 1024, 4, 96)
    for op in ("softmax", "softmax_bf16"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 128256, vocab) == RR_OK
    for op in ("rmsnorm", "layernorm", "residual_layernorm", "sum", "cross_entropy", "rmsnorm_bf16"):
        assert L.rr_check_plan(_capi.OP_IDS[op], 3, 128256, vocab) == RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(_capi.OP_IDS["softmax"], 3, 128256, plan(RR_PATH_LOOP, 256, 256, 4, 96)) == \
        RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(_capi.OP_IDS["softmax"], 3, 128256, plan(RR_PATH_LOOP, 1024, 1024, 2, 96)) == \
        RR_ERR_UNSUPPORTED


def test_v_wider_than_row_is_rejected(L):
    assert L.rr_check_plan(0, 1, 3, plan(RR_PATH_PACKED, 64, 8, 4, 4)) == RR_ERR_UNSUPPORTED
    assert L.rr_check_plan(0, 1, 3, plan(RR_PATH_PACKED, 64, 8, 2, 2)) == RR_OK


def test_check_plan_argument_errors(L):
    good = plan(RR_PATH_ROW, 256, 256, 4, 16)
    assert L.rr_check_plan(0, 64, 4096, good) == RR_OK
    for cache in (0, 1, 2):
        good.cache = cache
        assert L.rr_check_plan(0, 64, 4096, good) == RR_OK
    assert L.rr_check_plan(12, 64, 4096, good) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_check_plan(0, 64, 0, good) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_check_plan(0, 64, 4096, None) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_select_plan(12, 1, 1, rr_plan()) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_select_plan(0, 1, 1, None) == RR_ERR_INVALID_ARGUMENT


SHAPES = [(1, 1), (1, 2), (1, 3), (5, 31), (5, 33), (1, 127), (5, 128), (5, 129), (17, 257),
          (5, 4103), (64, 4096), (1024, 4096), (16384, 8192), (3, 32768), (2, 32769), (2, 100000),
          (100000, 16), (0, 7)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("op", OPS)
def test_selected_plans_are_legal_and_cover_the_row(L, op, rows, cols):
    p = rr_plan()
    assert L.rr_select_plan(_capi.OP_IDS[op], rows, cols, p) == RR_OK
    assert L.rr_check_plan(_capi.OP_IDS[op], rows, cols, p) == RR_OK
    assert p.rows_per_group * p.lanes_per_row == p.block
    if p.path != RR_PATH_LOOP:
        # The ownership map's private-slot bound fits the plan's registers.
        assert oracle.slot_bound(cols, p.lanes_per_row, p.v) <= p.slots
        assert p.lanes_per_row * p.slots >= cols
    else:
        assert cols > 1024 * 32
        assert p.slots in (0, 32, 64, 96)


def test_page_packing_arithmetic(L):
    """17 rows packed eight to a group need three groups (LuisaCompute page,
    "Result" section, the 17x257 remark)."""
    p = plan(RR_PATH_PACKED, 256, 32, 4, 16)
    assert p.rows_per_group == 8
    assert L.rr_check_plan(0, 17, 257, p) == RR_OK
    assert -(-17 // p.rows_per_group) == 3


def test_page_plans_are_expressible(L):
    """The page's worker / V choices map onto legal plans here (one row per
    group) with the slot count the ownership bound gives."""
    for rows, cols, workers, v in [(1, 127, 32, 4), (17, 257, 256, 4), (64, 4096, 128, 4),
                                   (1024, 4096, 256, 2)]:
        need = oracle.slot_bound(cols, workers, v)
        chunks = 1
        while chunks * v < need:
            chunks *= 2
        path = RR_PATH_PACKED if workers < 64 else RR_PATH_ROW
        block = max(64, workers)
        p = plan(path, block, workers, v, chunks * v)
        assert L.rr_check_plan(0, rows, cols, p) == RR_OK, (rows, cols, workers, v)


def test_algorithmic_bytes_table():
    """Byte counts of one call: each input read once, each output written once."""
    assert workloads.algorithmic_bytes("rmsnorm", 16384, 8192) == 1073774592
    assert workloads.algorithmic_bytes("rmsnorm", 1024, 4096) == 33570816
    assert workloads.algorithmic_bytes("sum", 1024, 4096) == 16781312
    assert workloads.algorithmic_bytes("residual_layernorm", 64, 4096) == 3178496
    assert workloads.algorithmic_bytes("cross_entropy", 17, 257) == 17612


# ---------------------------------------------------------------- split rows

def split(lanes, v, slots, cache=2):
    return rr_plan(RR_PATH_SPLIT, lanes, lanes, 1, v, slots, cache)


def test_split_plan_legality(L):
    rms, rms16 = 0, _capi.OP_IDS["rmsnorm_bf16"]
    assert L.rr_check_plan(rms, 2, 100003, split(256, 4, 16)) == RR_OK           # 25 slices
    assert L.rr_check_plan(rms, 2, 4096, split(256, 4, 16)) == RR_ERR_UNSUPPORTED   # one slice
    assert L.rr_check_plan(rms, 2, 100003, split(256, 2, 16)) == RR_ERR_UNSUPPORTED  # V must be 4
    assert L.rr_check_plan(rms, 2, 100003, split(256, 4, 8)) == RR_ERR_UNSUPPORTED   # slots 16 or 32
    assert L.rr_check_plan(rms, 2, 100003, split(256, 4, 16, 0)) == RR_ERR_UNSUPPORTED  # cache 2
    assert L.rr_check_plan(rms, 2, 100003, split(32, 4, 16)) == RR_ERR_UNSUPPORTED   # >= 64 lanes
    assert L.rr_check_plan(rms, 2, 64 * 16 * 1025, split(64, 4, 16)) == RR_ERR_UNSUPPORTED  # > 1024 slices
    assert L.rr_check_plan(rms, 70000, 100003, split(256, 4, 16)) == RR_ERR_UNSUPPORTED  # rows > 65535
    assert L.rr_check_plan(rms16, 2, 100000, split(256, 8, 16)) == RR_OK
    assert L.rr_check_plan(rms16, 2, 100003, split(256, 8, 16)) == RR_ERR_UNSUPPORTED  # cols % 8


def test_workspace_bytes(L):
    p = split(256, 4, 16)
    assert L.rr_workspace_bytes(0, 3, 100003, p) == 3 * 25 * 16
    assert L.rr_workspace_bytes(0, 3, 4096, plan(RR_PATH_ROW, 256, 256, 4, 16)) == 0
    assert L.rr_workspace_bytes(0, 3, 4096, p) == -1                  # illegal plan
    # Selector with unlimited workspace: few long rows split (64-lane slices of
    # 1024 columns here), many rows and short rows do not.
    assert L.rr_workspace_bytes(0, 3, 100003, None) == 3 * 98 * 16
    assert L.rr_workspace_bytes(0, 4096, 100003, None) == 0
    assert L.rr_workspace_bytes(0, 3, 4096, None) == 0
    assert L.rr_workspace_bytes(99, 3, 4096, None) == -1


def test_split_needs_workspace_and_alignment(L):
    p = split(256, 4, 16)
    assert L.rmsnorm_f32_ex(P, P, P, 3, 100003, 1e-6, p, None) == RR_ERR_UNSUPPORTED
    assert L.rmsnorm_f32_ws(P, P, P, 3, 100003, 1e-6, p, P, 3 * 25 * 16 - 1, None) == RR_ERR_UNSUPPORTED
    assert L.rmsnorm_f32_ws(P, P, P, 3, 100003, 1e-6, p, ctypes.c_void_p(0x10008), 4096, None) == \
        RR_ERR_INVALID_ARGUMENT                                       # workspace not 16-byte aligned
    assert L.rmsnorm_f32_ws(P, P, P, 3, 100003, 1e-6, None, P, -1, None) == RR_ERR_INVALID_ARGUMENT
    assert L.cross_entropy_f32_ws(P, P, P, 3, 100003, p, None, 0, None) == RR_ERR_UNSUPPORTED


# ---------------------------------------------------------------- batched launch (no launch happens)

def test_batch_argument_errors(L):
    from row_reduction_amd._capi import RR_BATCH_MAX, rr_problem
    arr = (rr_problem * (RR_BATCH_MAX + 1))()
    assert L.rr_batch(arr, -1, None) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_batch(arr, RR_BATCH_MAX + 1, None) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_batch(None, 1, None) == RR_ERR_INVALID_ARGUMENT
    assert L.rr_batch(None, 0, None) == RR_OK        # nothing to do
    # Zero-row problems are skipped without looking at their pointers.
    for i in range(3):
        arr[i].op, arr[i].rows, arr[i].cols = i, 0, 8
    assert L.rr_batch(arr, 3, None) == RR_OK
    # One invalid problem fails the whole batch before anything launches.
    good = rr_problem(op=0, eps=1e-6, rows=4, cols=8, x=0x1000, w=0x2000, y=0x3000)
    bad_eps = rr_problem(op=0, eps=-1.0, rows=4, cols=8, x=0x1000, w=0x2000, y=0x3000)
    missing = rr_problem(op=1, rows=4, cols=8, x=0x1000)                 # row sum without `out`
    unaligned = rr_problem(op=2, rows=4, cols=8, x=0x1002, y=0x3000)     # float x at 2 bytes
    unknown = rr_problem(op=12, rows=4, cols=8, x=0x1000, y=0x3000)
    neg_cols = rr_problem(op=2, rows=4, cols=0, x=0x1000, y=0x3000)
    for bad in (bad_eps, missing, unaligned, unknown, neg_cols):
        two = (rr_problem * 2)(good, bad)
        assert L.rr_batch(two, 2, None) == RR_ERR_INVALID_ARGUMENT
    too_wide = rr_problem(op=2, rows=4, cols=1 << 31, x=0x1000, y=0x3000)
    assert L.rr_batch((rr_problem * 1)(too_wide), 1, None) == RR_ERR_UNSUPPORTED
    # More than 2^31 - 1 workgroups in total (four short rows per group): refused,
    # nothing launched.
    big = rr_problem(op=1, rows=(1 << 32) + 1, cols=1, x=0x1000, row_out=0x2000)
    assert L.rr_batch((rr_problem * 2)(big, big), 2, None) == RR_ERR_UNSUPPORTED

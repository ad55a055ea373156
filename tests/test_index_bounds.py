"""Memory safety of the kernels' addressing, checked on the host.

A model of the index arithmetic the kernels use (consecutive-worker ownership
i = (chunk * W + lane) * V + e, the in-bounds window load at
min(i0, cols - V) whose slots keep only columns >= i0, the guarded store, the
slice bounds of split rows, the kept chunks of the streaming path) is run
for every legal plan the library accepts on many shapes. For each it checks
that every load lies inside the row, that the values a row's reduction uses
are exactly its columns, each once, and that every column is stored exactly
once, by the lane that read it. Plans come from the library's own legality
check (rr_check_plan), so a plan it accepts but this model would refuse
fails here."""
import numpy as np
import pytest

import row_reduction_amd as rr
from row_reduction_amd import _capi, plans
from row_reduction_amd._capi import RR_OK, rr_plan

RNG = np.random.default_rng(11)
COLS = sorted({1, 2, 3, 4, 5, 7, 8, 9, 31, 33, 63, 64, 65, 127, 128, 129, 255, 257, 1000, 1023, 1024, 1025,
               4095, 4096, 4097, 8191, 8192, 12289, 32767, 32768, 32769, 40000, 65536, 65537}
              | set(int(c) for c in RNG.integers(1, 70000, 12)))


def window(i0, cols, v):
    """(start, kept-columns mask) of the pack at i0 (numpy arrays over lanes)."""
    start = np.minimum(i0, cols - v)
    e = np.arange(v)
    cols_ = start[:, None] + e[None, :]
    keep = cols_ >= i0[:, None]
    return start, cols_, keep


def store_cols(i0, cols, end, v):
    """Columns the guarded store writes for packs at i0 (row end `cols`,
    slice end `end`): the whole pack when it ends by `end`, else the pack's
    own window columns before `end`."""
    start, cols_, keep = window(i0, cols, v)
    complete = (i0 + v) <= end
    out = np.where(complete[:, None], i0[:, None] + np.arange(v)[None, :], cols_)
    mask = np.where(complete[:, None], True, keep & (cols_ < end))
    return out, mask


def check_pass(cols, lanes, v, chunks, first=0, end=None):
    """Loads, kept values and stores of `chunks` packs per lane of one row
    (or one slice [first, end)); returns kept and stored column lists."""
    end = cols if end is None else end
    lane = np.arange(lanes)
    kept_all, stored_all = [], []
    for c in range(chunks):
        i0 = c * lanes * v + first + lane * v
        start, cols_, keep = window(i0, cols, v)
        assert (start >= 0).all() and (start + v <= cols).all(), "load outside the row"
        use = keep & (cols_ < end)
        kept_all.append(cols_[use])
        out, mask = store_cols(i0, cols, end, v)
        stored = out[mask]
        assert (stored >= 0).all() and (stored < cols).all(), "store outside the row"
        # Every stored column was read (and kept) by the same lane in the same pack.
        assert np.array_equal(np.sort(stored), np.sort(cols_[use])), "store of a column not kept"
        stored_all.append(stored)
    return np.concatenate(kept_all), np.concatenate(stored_all)


def assert_each_once(values, lo, hi, what):
    values = np.sort(values)
    assert np.array_equal(values, np.arange(lo, hi)), what


def register_plans(op, rows, cols):
    out = []
    for p in plans.candidate_plans(op, rows, cols, include_loop=False):
        out.append(p)
    return out


@pytest.mark.parametrize("op", ["rmsnorm", "softmax_bf16"])
def test_register_paths_read_and_write_each_column_once(op):
    n = 0
    for cols in COLS:
        for p in register_plans(op, 5, cols):
            exact = p.lanes_per_row * p.slots == cols
            kept, stored = check_pass(cols, p.lanes_per_row, p.v, p.slots // p.v)
            assert_each_once(kept, 0, cols, f"{op} {cols} {plans.plan_key(p)} kept")
            assert_each_once(stored, 0, cols, f"{op} {cols} {plans.plan_key(p)} stored")
            if exact:
                # Exact instances load without windows: every pack is complete.
                i0 = np.arange(p.slots // p.v)[:, None] * p.lanes_per_row * p.v + np.arange(p.lanes_per_row) * p.v
                assert (i0 + p.v <= cols).all()
            n += 1
    assert n > 200


@pytest.mark.parametrize("op", ["rmsnorm", "softmax", "layernorm_bf16", "sum"])
def test_streaming_path_with_kept_chunks(op):
    """Kept chunks (registers) then streamed chunks: every chunk index the
    kernel touches, including kept chunks past the row's last, is in bounds;
    the union is each column once."""
    n = 0
    for cols in COLS:
        for block in (64, 256, 1024):
            for v in (1, 2, 4, 8):
                for kept_slots in (0, 32, 64):
                    p = rr_plan(2, block, block, 1, v, kept_slots, 2)
                    if rr.rr_check_plan(op, 3, cols, p) != RR_OK:
                        continue
                    nchunk = -(-cols // (block * v))
                    keep = kept_slots // v
                    touched = max(nchunk, keep)          # kept chunks are loaded even past the row
                    kept, stored = check_pass(cols, block, v, touched)
                    assert_each_once(kept, 0, cols, f"{op} {cols} {plans.plan_key(p)}")
                    assert_each_once(stored, 0, cols, f"{op} {cols} {plans.plan_key(p)} stored")
                    n += 1
    assert n > 100


@pytest.mark.parametrize("op", ["rmsnorm", "softmax_bf16", "layernorm"])
def test_split_slices_partition_the_row(op):
    n = 0
    for cols in [c for c in COLS if c >= 8192] + [100003, 1 << 20, (1 << 20) + 8]:
        for lanes, slots in ((256, 16), (256, 32), (1024, 32), (64, 16)):
            v = 8 if op.endswith("_bf16") else 4
            p = rr_plan(3, lanes, lanes, 1, v, slots, 2)
            if rr.rr_check_plan(op, 2, cols, p) != RR_OK:
                continue
            span = lanes * slots
            slices = -(-cols // span)
            kept_all, stored_all = [], []
            for s in range(slices):
                first = s * span
                end = min(first + span, cols)
                kept, stored = check_pass(cols, lanes, v, slots // v, first, end)
                assert ((kept >= first) & (kept < end)).all()
                kept_all.append(kept)
                stored_all.append(stored)
            assert_each_once(np.concatenate(kept_all), 0, cols, f"split {op} {cols} {lanes}x{slots}")
            assert_each_once(np.concatenate(stored_all), 0, cols, f"split {op} {cols} {lanes}x{slots} stored")
            assert rr.rr_workspace_bytes(op, 2, cols, p) == 2 * slices * 16
            n += 1
    assert n > 20


def test_packed_groups_never_touch_rows_past_the_end():
    """Rows of a group past the last row mirror the last row and store
    nothing: the grid covers every row once."""
    for rows in (1, 7, 8, 9, 1003):
        for lanes in (8, 16, 32):
            for block in (64, 256):
                R = block // lanes
                groups = -(-rows // R)
                row_raw = np.arange(groups)[:, None] * R + np.arange(R)[None, :]
                row_ok = row_raw < rows
                row = np.where(row_ok, row_raw, rows - 1)
                assert (row >= 0).all() and (row < rows).all()
                assert np.array_equal(np.sort(row_raw[row_ok]), np.arange(rows))


def test_batch_groups_map_to_rows_of_one_problem():
    """rr_batch's (group, wavefront) -> (problem, row) map: problem i owns
    groups [first_i, first_i + ceil(rows_i / R_i)) with R_i = 256 / lanes_i
    rows per group (lanes 64 below 2048 columns, else 256); each of its rows
    is served once, and wavefronts past its last row exit (only with one
    wavefront per row, where no barrier follows)."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        count = int(rng.integers(1, _capi.RR_BATCH_MAX + 1))
        rows = rng.integers(0, 40, count)
        cols = rng.choice([7, 100, 2047, 2048, 5000], count)
        keep = rows > 0
        rows, cols = rows[keep], cols[keep]
        if rows.size == 0:
            continue
        lanes = np.where(cols >= 2048, 256, 64)
        per_group = 256 // lanes
        groups = -(-rows // per_group)
        first = np.concatenate([[0], np.cumsum(groups)[:-1]])
        seen = []
        for blk in range(int(groups.sum())):
            i = 0
            while i + 1 < rows.size and first[i + 1] <= blk:
                i += 1
            for tid in range(0, 256, 64):          # one wavefront at a time
                r = (blk - first[i]) * per_group[i] + (tid >> (8 if lanes[i] == 256 else 6))
                if r >= rows[i]:
                    assert lanes[i] == 64           # an exiting wavefront never has barrier partners
                    continue
                if lanes[i] == 256 and tid > 0:
                    continue                        # the same row: counted once per group
                seen.append((i, int(r)))
        assert len(seen) == len(set(seen)) == int(rows.sum())


def test_widest_rows_keep_every_index_in_32_bits():
    """Kernels form column indices in 32-bit ints: for the widest accepted
    row and every legal streaming plan, the largest index any lane forms
    (pack starts of every chunk touched, including kept chunks, plus the
    chunk-count rounding cols + stride - 1) stays below 2^31; one column
    more is refused."""
    cols = _capi.RR_MAX_COLS
    L = _capi.lib()
    for op in _capi.OP_IDS:
        assert rr.rr_check_plan(op, 1, cols + 1, rr.rr_select_plan(op, 1, 8)) == _capi.RR_ERR_UNSUPPORTED
        p = rr.rr_select_plan(op, 1, cols)
        assert rr.rr_check_plan(op, 1, cols, p) == RR_OK
        assert L.rr_select_plan(_capi.OP_IDS[op], 1, cols + 1, rr_plan()) == _capi.RR_ERR_UNSUPPORTED
    n = 0
    for op in ("rmsnorm", "softmax", "layernorm", "sum_bf16", "softmax_bf16"):
        for block in (64, 256, 1024):
            for v in (1, 2, 4, 8):
                for kept in (0, 32, 64):
                    p = rr_plan(2, block, block, 1, v, kept, 2)
                    if rr.rr_check_plan(op, 1, cols, p) != RR_OK:
                        continue
                    stride = block * v
                    nchunk = (cols + stride - 1) // stride
                    assert cols + stride - 1 < 2 ** 31
                    last_chunk = max(nchunk, kept // v + 32 // v) - 1   # kept and LDS-kept chunks
                    biggest = last_chunk * stride + (block - 1) * v + v
                    assert biggest < 2 ** 31, (op, plans.plan_key(p), biggest)
                    n += 1
    assert n > 20


def stream_kernel_accesses(n, packs_per_thread, block):
    """Host model of rr_stream_f32's indexing: (grid, packs read per thread,
    tail floats) exactly as the kernel forms them."""
    packs = n // 4
    groups = max(1, -(-packs // (packs_per_thread * block)))
    touched = []
    for g in range(groups):
        for t in range(block):
            first = g * packs_per_thread * block + t
            if first + (packs_per_thread - 1) * block < packs:
                touched += [first + u * block for u in range(packs_per_thread)]
            else:
                u = 0
                while u < packs_per_thread and first + u * block < packs:
                    touched.append(first + u * block)
                    u += 1
    tail = [4 * packs + t for t in range(block) if t < (n & 3)]
    return groups, touched, tail


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 4096, 4099, 65536 + 7, 300001])
@pytest.mark.parametrize("packs_per_thread", [1, 2, 4, 8])
@pytest.mark.parametrize("block", [256, 512, 1024])
def test_stream_kernel_covers_every_float_once_in_bounds(n, packs_per_thread, block):
    groups, touched, tail = stream_kernel_accesses(n, packs_per_thread, block)
    assert sorted(touched) == list(range(n // 4)), "every whole pack exactly once"
    assert all(4 * p + 3 < n for p in touched), "no pack past the end"
    assert tail == list(range(4 * (n // 4), n)), "trailing floats exactly once"
    # Read-only form: the never-taken sink index stays inside groups * block floats.
    assert groups * block >= 1

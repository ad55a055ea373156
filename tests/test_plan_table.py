"""The frozen plan table was measured on the device sources the library is
built from. Each entry carries the start of the sha256 of the device sources
it was timed under; a kernel change after the search would leave timings of
other kernels frozen in the table, so every stamp must equal the current
sources' hash (else: run the search and replay again, then emit the table)."""
import os
import re

from row_reduction_amd import _capi
from row_reduction_amd.tune import DEFAULT_SHAPES, source_hash

TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "row_reduction_amd", "csrc", "plan_table.inc")


def entries():
    return [ln for ln in open(TABLE).read().splitlines() if ln.startswith("{")]


def test_every_entry_is_stamped_with_the_current_device_sources():
    cur = source_hash()[:8]
    stale = []
    for ln in entries():
        m = re.search(r"// \[([0-9a-f]{8})\]", ln)
        assert m, f"entry without a source stamp: {ln}"
        if m.group(1) != cur:
            stale.append(ln)
    assert not stale, (f"{len(stale)} table entries were measured under other device sources "
                       f"(current {cur}); re-run the plan search and replay, then emit the table:\n"
                       + "\n".join(stale[:5]))


def test_table_lists_every_operator_on_every_measured_shape_once():
    keys = []
    for ln in entries():
        op, rows, cols = (int(v) for v in ln[1:].split(",")[:3])
        keys.append((op, rows, cols))
    assert len(keys) == len(set(keys))
    want = {(op, *map(int, s.split("x"))) for op in set(_capi.OP_IDS.values()) for s in DEFAULT_SHAPES}
    assert set(keys) == want

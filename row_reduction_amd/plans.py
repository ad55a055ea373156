"""Enumeration of legal launch plans for one (op, rows, cols).

The finite search space of the plan selector: which row-to-workgroup family
(several rows per wavefront, whole wavefronts per row, or the streaming
loop), how many workers share a row and how many consecutive floats each
owns per pack. Candidates are generated first and filtered through the
library's own legality check, so an illegal candidate is never timed
(LuisaCompute notes, "Consecutive-worker reduction layout checkpoint",
section "Implementation and semantics": the private-storage bound is enforced
before any scoring).
"""
from __future__ import annotations

from . import _capi
from ._capi import RR_OK, RR_PATH_LOOP, RR_PATH_PACKED, RR_PATH_ROW, RR_PATH_SPLIT, rr_plan

PACKED_LANES = (8, 16, 32)
PACKED_BLOCKS = (64, 256)
ROW_LANES = (64, 128, 256, 512, 1024)
VS = (1, 2, 4)
VS_BF16 = (1, 2, 4, 8)
CHUNKS = (1, 2, 4, 8)
LOOP_BLOCKS = (256, 1024)
LOOP_KEPT_SLOTS = (0, 32, 64, 96)   # streaming: register slots kept between the two passes
CACHES = (0, 1, 2)


def _min_chunks(cols: int, lanes: int, v: int):
    for c in CHUNKS:
        if lanes * v * c >= cols:
            return c
    return None


def candidate_plans(op: str, rows: int, cols: int, include_loop: bool = True,
                    caches=(0,)) -> list[rr_plan]:
    """Every legal plan of the search grid, with the fewest chunks that cover a
    row, for each cache policy in `caches`."""
    op_id = _capi.OP_IDS[op]
    L = _capi.lib()
    out = []

    def add(p: rr_plan):
        for cache in caches:
            q = rr_plan.from_dict({**p.as_dict(), "cache": cache})
            if L.rr_check_plan(op_id, rows, cols, q) == RR_OK:
                out.append(q)

    vs = VS_BF16 if op.endswith("_bf16") else VS
    for lanes in PACKED_LANES:
        for block in PACKED_BLOCKS:
            for v in vs:
                c = _min_chunks(cols, lanes, v)
                if c is not None:
                    add(rr_plan(RR_PATH_PACKED, block, lanes, block // lanes, v, c * v))
    for lanes in ROW_LANES:
        blocks = sorted({lanes, max(lanes, 256)})
        for block in blocks:
            for v in vs:
                c = _min_chunks(cols, lanes, v)
                if c is not None:
                    add(rr_plan(RR_PATH_ROW, block, lanes, block // lanes, v, c * v))
    if include_loop:
        for block in LOOP_BLOCKS:
            for v in vs:
                for kept in LOOP_KEPT_SLOTS:
                    add(rr_plan(RR_PATH_LOOP, block, block, 1, v, kept))
    return out


def plan_key(p: rr_plan) -> str:
    name = {RR_PATH_PACKED: "packed", RR_PATH_ROW: "row", RR_PATH_LOOP: "loop", RR_PATH_SPLIT: "split"}[p.path]
    return f"{name}-b{p.block}-w{p.lanes_per_row}-v{p.v}-k{p.slots}-c{p.cache}"

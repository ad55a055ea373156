"""Host-side reentrancy (CPU): the planner's calls, made from several host
threads at once (ctypes releases the GIL for the call), return exactly what
the same calls return one at a time; this exercises the mutex-guarded cache
of the model's recent choices under contention."""
import threading

import numpy as np

from row_reduction_amd import _capi
from row_reduction_amd._capi import rr_plan


def shapes(seed, n):
    rng = np.random.default_rng(seed)
    rows = np.round(2 ** rng.uniform(0, 16, n)).astype(np.int64)
    cols = np.round(2 ** rng.uniform(0, 20, n)).astype(np.int64)
    ops = rng.integers(0, 12, n)
    return list(zip(ops.tolist(), rows.tolist(), cols.tolist()))


def plan_of(L, op, rows, cols):
    p = rr_plan()
    st = L.rr_select_plan(op, rows, cols, p)
    return st, tuple(p.as_dict().values()), L.rr_workspace_bytes(op, rows, cols, None)


def test_concurrent_selection_equals_sequential():
    L = _capi.lib()
    work = shapes(5, 600)
    # Few distinct shapes repeated many times keep the model's cache busy
    # with hits, misses and evictions from every thread at once.
    work = work + work[:40] * 10
    want = [plan_of(L, *w) for w in work]
    got = {}
    errors = []

    def worker(t):
        try:
            order = np.random.default_rng(t).permutation(len(work))
            got[t] = {int(i): plan_of(L, *work[int(i)]) for i in order}
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(8):
        for i, w in enumerate(want):
            assert got[t][i] == w, (t, work[i], got[t][i], w)

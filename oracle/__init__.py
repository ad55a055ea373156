"""CPU oracle for the FP32 row-reduction family — test infrastructure only.

Wraps ``oracle.c`` (plain fp64 C loops, one rounding to float32 per output)
with numpy-in / numpy-out functions. Only ``tests/``, the package smoke check
and the benchmark's CPU-baseline leg may import this package; the product
path never does, and this package imports nothing from the product.

Each function states the definition it computes; ``oracle.c`` cites the page
passage each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

# ORACLE_LIB names another build of oracle.c to load instead (the tests that
# plant mistakes in a copy of the source and check that the pins catch them).
_OVERRIDE = os.environ.get("ORACLE_LIB")


def _load():
    global _lib
    if _lib is None:
        if _OVERRIDE is None and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_OVERRIDE or _LIB)
        lib.oracle_rmsnorm_f32.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, ctypes.c_float]
        lib.oracle_rmsnorm_f32_sampled.argtypes = [_f32p, _f32p, _i64, ctypes.c_float, _i64p, _i64, _f32p]
        lib.oracle_row_sum_f32_long.argtypes = [_f32p, _i64, _f32p]
        lib.oracle_softmax_f32_sampled.argtypes = [_f32p, _i64, _i64p, _i64, _f32p]
        lib.oracle_row_sum_f32.argtypes = [_f32p, _f32p, _i64, _i64]
        lib.oracle_softmax_f32.argtypes = [_f32p, _f32p, _i64, _i64]
        lib.oracle_layernorm_f32.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, ctypes.c_float]
        lib.oracle_residual_layernorm_f32.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p,
                                                      _i64, _i64, ctypes.c_float]
        lib.oracle_cross_entropy_f32.argtypes = [_f32p, _i32p, _f32p, _i64, _i64]
        lib.oracle_rmsnorm_bf16.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, ctypes.c_float]
        lib.oracle_row_sum_bf16.argtypes = [_u16p, _f32p, _i64, _i64]
        lib.oracle_softmax_bf16.argtypes = [_u16p, _u16p, _i64, _i64]
        lib.oracle_layernorm_bf16.argtypes = [_u16p, _u16p, _u16p, _u16p, _i64, _i64, ctypes.c_float]
        lib.oracle_residual_layernorm_bf16.argtypes = [_u16p, _u16p, _u16p, _u16p, _u16p, _u16p,
                                                       _i64, _i64, ctypes.c_float]
        lib.oracle_cross_entropy_bf16.argtypes = [_u16p, _i32p, _f32p, _i64, _i64]
        lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        lib.oracle_owner.argtypes = [_i64, _i64, _i64, _i64p, _i64p]
        lib.oracle_owner.restype = None
        lib.oracle_logical_index.argtypes = [_i64, _i64, _i64, _i64]
        lib.oracle_logical_index.restype = _i64
        lib.oracle_slot_bound.argtypes = [_i64, _i64, _i64]
        lib.oracle_slot_bound.restype = _i64
        _lib = lib
    return _lib


def _f32(a, ndim):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != ndim:
        raise ValueError(f"expected {ndim}-d array, got shape {a.shape}")
    return a


def _p(a, t):
    return a.ctypes.data_as(t)


def _check(rc):
    if rc == 2:
        raise MemoryError("oracle scratch allocation failed")
    if rc != 0:
        raise ValueError("oracle rejected the arguments (rows < 0 or cols <= 0)")


def rmsnorm(x, w, eps):
    """y[r,c] = x[r,c]*w[c] / sqrt(mean_c x[r,c]^2 + eps)."""
    x = _f32(x, 2)
    w = _f32(w, 1)
    rows, cols = x.shape
    assert w.shape == (cols,)
    y = np.empty_like(x)
    _check(_load().oracle_rmsnorm_f32(_p(x, _f32p), _p(w, _f32p), _p(y, _f32p), rows, cols, eps))
    return y


def row_sum(x):
    """out[r] = sum_c x[r,c]."""
    x = _f32(x, 2)
    rows, cols = x.shape
    out = np.empty(rows, np.float32)
    _check(_load().oracle_row_sum_f32(_p(x, _f32p), _p(out, _f32p), rows, cols))
    return out


def softmax(x):
    """y[r,c] = exp(x[r,c]-m_r) / sum_k exp(x[r,k]-m_r), m_r the row maximum."""
    x = _f32(x, 2)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_softmax_f32(_p(x, _f32p), _p(y, _f32p), rows, cols))
    return y


def _row_and_idx(x, idx):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 1
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    return x, idx


def rmsnorm_sampled(x, w, eps, idx):
    """rmsnorm of the single row x (1-D float32, up to 2^31 columns) at the
    columns idx only; the row statistic covers the whole row."""
    x, idx = _row_and_idx(x, idx)
    w = _f32(w, 1)
    assert w.shape == x.shape
    y = np.empty(idx.size, np.float32)
    _check(_load().oracle_rmsnorm_f32_sampled(_p(x, _f32p), _p(w, _f32p), x.size, eps,
                                              _p(idx, _i64p), idx.size, _p(y, _f32p)))
    return y


def row_sum_long(x):
    """sum_c x[c] of the single row x (1-D float32), in float64, no row copy."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(1, np.float32)
    _check(_load().oracle_row_sum_f32_long(_p(x, _f32p), x.size, _p(out, _f32p)))
    return out[0]


def softmax_sampled(x, idx):
    """softmax of the single row x (1-D float32) at the columns idx only."""
    x, idx = _row_and_idx(x, idx)
    y = np.empty(idx.size, np.float32)
    _check(_load().oracle_softmax_f32_sampled(_p(x, _f32p), x.size, _p(idx, _i64p), idx.size,
                                              _p(y, _f32p)))
    return y


def layernorm(x, gamma, beta, eps):
    """y = (x-mean)/sqrt(var+eps)*gamma + beta, population variance per row."""
    x = _f32(x, 2)
    g = _f32(gamma, 1)
    b = _f32(beta, 1)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_layernorm_f32(_p(x, _f32p), _p(g, _f32p), _p(b, _f32p), _p(y, _f32p),
                                        rows, cols, eps))
    return y


def residual_layernorm(x, residual, gamma, beta, eps):
    """h = fl32(x + residual); y = LayerNorm(h). Returns (y, h)."""
    x = _f32(x, 2)
    r = _f32(residual, 2)
    g = _f32(gamma, 1)
    b = _f32(beta, 1)
    rows, cols = x.shape
    assert r.shape == x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    _check(_load().oracle_residual_layernorm_f32(_p(x, _f32p), _p(r, _f32p), _p(g, _f32p),
                                                 _p(b, _f32p), _p(y, _f32p), _p(h, _f32p),
                                                 rows, cols, eps))
    return y, h


def cross_entropy(logits, targets):
    """loss[r] = logsumexp_c x[r,c] - x[r,t[r]]; NaN for a target outside [0, cols)."""
    x = _f32(logits, 2)
    t = np.ascontiguousarray(targets, dtype=np.int32)
    rows, cols = x.shape
    assert t.shape == (rows,)
    loss = np.empty(rows, np.float32)
    _check(_load().oracle_cross_entropy_f32(_p(x, _f32p), _p(t, _i32p), _p(loss, _f32p), rows, cols))
    return loss


# ---- bfloat16 storage (arrays of uint16 bit patterns) -----------------------

def _u16(a, ndim):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bfloat16 data is passed as uint16 bit patterns")
    if a.ndim != ndim:
        raise ValueError(f"expected {ndim}-d array, got shape {a.shape}")
    return a


def bf16_from_double(v: float) -> int:
    """Bit pattern of the bfloat16 nearest to v (ties to even), rounded once."""
    return int(_load().oracle_bf16_from_double(float(v)))


def bf16_to_float(b) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rmsnorm_bf16(x, w, eps):
    x = _u16(x, 2)
    w = _u16(w, 1)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_rmsnorm_bf16(_p(x, _u16p), _p(w, _u16p), _p(y, _u16p), rows, cols, eps))
    return y


def row_sum_bf16(x):
    x = _u16(x, 2)
    rows, cols = x.shape
    out = np.empty(rows, np.float32)
    _check(_load().oracle_row_sum_bf16(_p(x, _u16p), _p(out, _f32p), rows, cols))
    return out


def softmax_bf16(x):
    x = _u16(x, 2)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_softmax_bf16(_p(x, _u16p), _p(y, _u16p), rows, cols))
    return y


def layernorm_bf16(x, gamma, beta, eps):
    x = _u16(x, 2)
    g = _u16(gamma, 1)
    b = _u16(beta, 1)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_layernorm_bf16(_p(x, _u16p), _p(g, _u16p), _p(b, _u16p), _p(y, _u16p),
                                         rows, cols, eps))
    return y


def residual_layernorm_bf16(x, residual, gamma, beta, eps):
    x = _u16(x, 2)
    r = _u16(residual, 2)
    g = _u16(gamma, 1)
    b = _u16(beta, 1)
    rows, cols = x.shape
    y = np.empty_like(x)
    h = np.empty_like(x)
    _check(_load().oracle_residual_layernorm_bf16(_p(x, _u16p), _p(r, _u16p), _p(g, _u16p),
                                                  _p(b, _u16p), _p(y, _u16p), _p(h, _u16p),
                                                  rows, cols, eps))
    return y, h


def cross_entropy_bf16(logits, targets):
    x = _u16(logits, 2)
    t = np.ascontiguousarray(targets, dtype=np.int32)
    rows, cols = x.shape
    loss = np.empty(rows, np.float32)
    _check(_load().oracle_cross_entropy_bf16(_p(x, _u16p), _p(t, _i32p), _p(loss, _f32p), rows, cols))
    return loss


def owner(i, W, V):
    """(worker, slot) of logical element i under W workers with V consecutive elements each."""
    wk = ctypes.c_int64()
    sl = ctypes.c_int64()
    _load().oracle_owner(i, W, V, ctypes.byref(wk), ctypes.byref(sl))
    return wk.value, sl.value


def logical_index(worker, slot, W, V):
    """Logical element held in private `slot` of `worker`."""
    return _load().oracle_logical_index(worker, slot, W, V)


def slot_bound(N, W, V):
    """Largest count of valid private slots of any worker for a row of N elements."""
    return _load().oracle_slot_bound(N, W, V)


def run(op: str, wl_arrays: dict):
    """Dispatch by operator name; `wl_arrays` holds x, w, beta, residual, targets, eps."""
    a = wl_arrays
    if op == "rmsnorm":
        return rmsnorm(a["x"], a["w"], a["eps"])
    if op == "sum":
        return row_sum(a["x"])
    if op == "softmax":
        return softmax(a["x"])
    if op == "layernorm":
        return layernorm(a["x"], a["w"], a["beta"], a["eps"])
    if op == "residual_layernorm":
        return residual_layernorm(a["x"], a["residual"], a["w"], a["beta"], a["eps"])
    if op == "cross_entropy":
        return cross_entropy(a["x"], a["targets"])
    raise ValueError(op)

"""ctypes view of librowred.so: the C entry points declared in include/rowred.h.

Loading fails loudly (RuntimeError) when the library has not been built;
there is no fallback implementation of any operator.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ROWRED_LIB selects another build of the library (e.g. one compiled with
# different streaming hints); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("ROWRED_LIB") or os.path.join(HERE, "librowred.so")

RR_OK = 0
RR_ERR_INVALID_ARGUMENT = 1
RR_ERR_UNSUPPORTED = 2
RR_ERR_LAUNCH = 3

RR_OP_RMSNORM = 0
RR_OP_SUM = 1
RR_OP_SOFTMAX = 2
RR_OP_LAYERNORM = 3
RR_OP_RESIDUAL_LAYERNORM = 4
RR_OP_CROSS_ENTROPY = 5
RR_OP_BF16_OFFSET = 6   # RR_OP_<op>_BF16 = RR_OP_<op> + 6

RR_PATH_PACKED = 0
RR_PATH_ROW = 1
RR_PATH_LOOP = 2
RR_PATH_SPLIT = 3

OP_IDS = {
    "rmsnorm": RR_OP_RMSNORM,
    "sum": RR_OP_SUM,
    "softmax": RR_OP_SOFTMAX,
    "layernorm": RR_OP_LAYERNORM,
    "residual_layernorm": RR_OP_RESIDUAL_LAYERNORM,
    "cross_entropy": RR_OP_CROSS_ENTROPY,
}
OP_IDS.update({f"{k}_bf16": v + RR_OP_BF16_OFFSET for k, v in list(OP_IDS.items())})

# Every symbol include/rowred.h declares.
EXPORTED = (
    "rmsnorm_f32", "row_sum_f32", "softmax_f32", "layernorm_f32",
    "residual_layernorm_f32", "cross_entropy_f32",
    "rmsnorm_f32_ex", "row_sum_f32_ex", "softmax_f32_ex", "layernorm_f32_ex",
    "residual_layernorm_f32_ex", "cross_entropy_f32_ex",
    "rmsnorm_bf16", "row_sum_bf16", "softmax_bf16", "layernorm_bf16",
    "residual_layernorm_bf16", "cross_entropy_bf16",
    "rmsnorm_bf16_ex", "row_sum_bf16_ex", "softmax_bf16_ex", "layernorm_bf16_ex",
    "residual_layernorm_bf16_ex", "cross_entropy_bf16_ex",
    "rmsnorm_f32_ws", "row_sum_f32_ws", "softmax_f32_ws", "layernorm_f32_ws",
    "residual_layernorm_f32_ws", "cross_entropy_f32_ws",
    "rmsnorm_bf16_ws", "row_sum_bf16_ws", "softmax_bf16_ws", "layernorm_bf16_ws",
    "residual_layernorm_bf16_ws", "cross_entropy_bf16_ws",
    "rr_workspace_bytes", "rmsnorm_f32_noalloc",
    "rr_select_plan", "rr_check_plan", "rr_status_string",
    "rr_select_plan_from", "rr_model_time_us", "rr_batch",
    "rr_copy_f32", "rr_stream_f32", "rr_empty_kernel",
)

# rr_plan_source
RR_PLAN_AUTO, RR_PLAN_TABLE, RR_PLAN_MODEL, RR_PLAN_RULE = 0, 1, 2, 3


class rr_plan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("v", ctypes.c_int32),
        ("slots", ctypes.c_int32),
        ("cache", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}

    @classmethod
    def from_dict(cls, d: dict) -> "rr_plan":
        return cls(**{name: int(d.get(name, 0)) for name, _ in cls._fields_})

    def __repr__(self) -> str:
        return f"rr_plan({self.as_dict()})"


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_planp = ctypes.POINTER(rr_plan)

RR_BATCH_MAX = 32
RR_MAX_COLS = (1 << 31) - (1 << 20)   # widest row (every kernel index fits in 32 bits)
RR_NOALLOC_SCRATCH_BYTES = 1 << 20   # rmsnorm_f32_noalloc's static split-row buffer


class rr_problem(ctypes.Structure):
    """One problem of rr_batch (include/rowred.h)."""
    _fields_ = [
        ("op", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("x", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
        ("w", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("targets", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("h_out", ctypes.c_void_p),
        ("row_out", ctypes.c_void_p),
    ]


_SIGNATURES = {
    "rmsnorm_f32": [_vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "row_sum_f32": [_vp, _vp, _i64, _i64, _vp],
    "softmax_f32": [_vp, _vp, _i64, _i64, _vp],
    "layernorm_f32": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "residual_layernorm_f32": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "cross_entropy_f32": [_vp, _vp, _vp, _i64, _i64, _vp],
    "rmsnorm_f32_ex": [_vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "row_sum_f32_ex": [_vp, _vp, _i64, _i64, _planp, _vp],
    "softmax_f32_ex": [_vp, _vp, _i64, _i64, _planp, _vp],
    "layernorm_f32_ex": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "residual_layernorm_f32_ex": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "cross_entropy_f32_ex": [_vp, _vp, _vp, _i64, _i64, _planp, _vp],
    "rmsnorm_bf16": [_vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "row_sum_bf16": [_vp, _vp, _i64, _i64, _vp],
    "softmax_bf16": [_vp, _vp, _i64, _i64, _vp],
    "layernorm_bf16": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "residual_layernorm_bf16": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
    "cross_entropy_bf16": [_vp, _vp, _vp, _i64, _i64, _vp],
    "rmsnorm_bf16_ex": [_vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "row_sum_bf16_ex": [_vp, _vp, _i64, _i64, _planp, _vp],
    "softmax_bf16_ex": [_vp, _vp, _i64, _i64, _planp, _vp],
    "layernorm_bf16_ex": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "residual_layernorm_bf16_ex": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "cross_entropy_bf16_ex": [_vp, _vp, _vp, _i64, _i64, _planp, _vp],
    "rmsnorm_f32_ws": [_vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "row_sum_f32_ws": [_vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "softmax_f32_ws": [_vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "layernorm_f32_ws": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "residual_layernorm_f32_ws": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "cross_entropy_f32_ws": [_vp, _vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "rmsnorm_bf16_ws": [_vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "row_sum_bf16_ws": [_vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "softmax_bf16_ws": [_vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "layernorm_bf16_ws": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "residual_layernorm_bf16_ws": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp, _i64, _vp],
    "cross_entropy_bf16_ws": [_vp, _vp, _vp, _i64, _i64, _planp, _vp, _i64, _vp],
    "rr_workspace_bytes": [ctypes.c_int, _i64, _i64, _planp],
    "rmsnorm_f32_noalloc": [_vp, _vp, _vp, _i64, _i64, _f32, _planp, _vp],
    "rr_select_plan": [ctypes.c_int, _i64, _i64, _planp],
    "rr_check_plan": [ctypes.c_int, _i64, _i64, _planp],
    "rr_select_plan_from": [ctypes.c_int, _i64, _i64, ctypes.c_int, _planp],
    "rr_model_time_us": [ctypes.c_int, _i64, _i64, _planp],
    "rr_batch": [ctypes.POINTER(rr_problem), ctypes.c_int32, _vp],
    "rr_status_string": [ctypes.c_int],
    "rr_copy_f32": [_vp, _vp, _i64, _vp],
    "rr_stream_f32": [_vp, _vp, _i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp],
    "rr_empty_kernel": [_vp],
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises RuntimeError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run "
                "`python row_reduction_amd/build.py` first")
        # torch ships its own HIP runtime under the same soname as ROCm's.
        # Loading torch first makes this library bind to that one runtime, so
        # the device pointers and stream handles torch hands over are valid
        # here. Loaded the other way round, the process would hold two HIP
        # runtimes and every launch on a torch stream would fail.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, argtypes in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = {"rr_status_string": ctypes.c_char_p,
                          "rr_workspace_bytes": ctypes.c_int64,
                          "rr_model_time_us": ctypes.c_double}.get(name, ctypes.c_int)
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().rr_status_string(code).decode()


class RowRedError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def check(fn: str, status: int) -> None:
    if status != RR_OK:
        raise RowRedError(fn, status)

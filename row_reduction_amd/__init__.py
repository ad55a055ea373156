"""FP32 row reductions on AMD Instinct MI355X (gfx950) — Python binding.

Thin wrappers over the C entry points of ``librowred.so`` (declared in
``include/rowred.h``) with the same names. They only marshal arguments:
check that tensors are contiguous float32 (int32 targets) on a GPU, pass
``data_ptr()`` values, the shape, and the current HIP stream, and allocate
outputs the caller did not supply. Every operator runs in the library's HIP
kernels; nothing here computes.

Importing this package does not load the library; the first call does, and
raises RuntimeError if it has not been built.
"""
from __future__ import annotations

from . import _capi
from ._capi import OP_IDS, RowRedError, rr_plan

__all__ = [
    "rmsnorm_f32", "row_sum_f32", "softmax_f32", "layernorm_f32",
    "residual_layernorm_f32", "cross_entropy_f32", "rmsnorm_f32_noalloc",
    "rmsnorm_bf16", "row_sum_bf16", "softmax_bf16", "layernorm_bf16",
    "residual_layernorm_bf16", "cross_entropy_bf16",
    "rr_select_plan", "rr_select_plan_from", "rr_model_time_us", "rr_check_plan", "rr_status_string",
    "rr_copy_f32", "rr_stream_f32", "rr_empty_kernel",
    "rr_workspace_bytes", "workspace_for", "batch_problem", "rr_batch",
    "rr_plan", "RowRedError", "OP_IDS",
]


def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is not None:
        return int(stream)
    return _torch().cuda.current_stream().cuda_stream


def _mat(t, name, dtype=None):
    torch = _torch()
    dtype = dtype or torch.float32
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} CUDA/HIP tensor")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-d tensor, got shape {tuple(t.shape)}")
    return t


def _vec(t, n, name, dtype=None):
    torch = _torch()
    dtype = dtype or torch.float32
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} CUDA/HIP tensor")
    if t.dim() != 1 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with {n} elements, got shape {tuple(t.shape)}")
    return t


def _out_like(out, x, name):
    if out is None:
        return _torch().empty_like(x)
    _mat(out, name, x.dtype)
    if out.shape != x.shape:
        raise ValueError(f"{name} must have shape {tuple(x.shape)}")
    return out


def _out_rows(out, x, name):
    torch = _torch()
    if out is None:
        return torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    return _vec(out, x.shape[0], name)


def _ws(workspace):
    """(pointer, bytes) of an optional workspace tensor (any dtype, on the GPU)."""
    if workspace is None:
        return None, 0
    torch = _torch()
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA/HIP tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def workspace_for(op, rows, cols, plan=None, device=None):
    """A workspace tensor large enough for `op` on (rows, cols) with `plan`
    (the selector's choice when None), or None when the plan needs none."""
    n = rr_workspace_bytes(op, rows, cols, plan)
    if n <= 0:
        return None
    torch = _torch()
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def _plan_ptr(plan):
    if plan is None:
        return None
    if isinstance(plan, dict):
        plan = rr_plan.from_dict(plan)
    return plan


def rmsnorm_f32(x, w, eps=1e-6, y=None, plan=None, workspace=None, stream=None):
    """y[r,c] = x[r,c] * w[c] / sqrt(mean_c x[r,c]^2 + eps). Returns y."""
    _mat(x, "x")
    rows, cols = x.shape
    _vec(w, cols, "w")
    y = _out_like(y, x, "y")
    st = _capi.lib().rmsnorm_f32_ws(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, cols, float(eps),
                                     _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("rmsnorm_f32", st)
    return y


def rmsnorm_f32_noalloc(x, w, eps=1e-6, y=None, plan=None, stream=None):
    """rmsnorm_f32 whose split-row partials use the library's static device
    buffer (no workspace, nothing allocated by the call when y is given).
    Calls on one GPU share that buffer: overlapping calls race. Returns y."""
    _mat(x, "x")
    rows, cols = x.shape
    _vec(w, cols, "w")
    y = _out_like(y, x, "y")
    st = _capi.lib().rmsnorm_f32_noalloc(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, cols, float(eps),
                                          _plan_ptr(plan), _stream(stream))
    _capi.check("rmsnorm_f32_noalloc", st)
    return y


def row_sum_f32(x, out=None, plan=None, workspace=None, stream=None):
    """out[r] = sum_c x[r,c] (float64 accumulation, one rounding). Returns out."""
    _mat(x, "x")
    rows, cols = x.shape
    out = _out_rows(out, x, "out")
    st = _capi.lib().row_sum_f32_ws(x.data_ptr(), out.data_ptr(), rows, cols, _plan_ptr(plan),
                                     *_ws(workspace), _stream(stream))
    _capi.check("row_sum_f32", st)
    return out


def softmax_f32(x, y=None, plan=None, workspace=None, stream=None):
    """Row softmax with the row maximum subtracted. Returns y."""
    _mat(x, "x")
    rows, cols = x.shape
    y = _out_like(y, x, "y")
    st = _capi.lib().softmax_f32_ws(x.data_ptr(), y.data_ptr(), rows, cols, _plan_ptr(plan),
                                     *_ws(workspace), _stream(stream))
    _capi.check("softmax_f32", st)
    return y


def layernorm_f32(x, gamma, beta, eps=1e-5, y=None, plan=None, workspace=None, stream=None):
    """y = (x - mean) / sqrt(var + eps) * gamma + beta per row. Returns y."""
    _mat(x, "x")
    rows, cols = x.shape
    _vec(gamma, cols, "gamma")
    _vec(beta, cols, "beta")
    y = _out_like(y, x, "y")
    st = _capi.lib().layernorm_f32_ws(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), y.data_ptr(),
                                       rows, cols, float(eps), _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("layernorm_f32", st)
    return y


def residual_layernorm_f32(x, residual, gamma, beta, eps=1e-5, y=None, h_out=None, plan=None,
                           workspace=None, stream=None):
    """h = x + residual (float32); y = LayerNorm(h). Writes h to h_out when given. Returns y."""
    _mat(x, "x")
    rows, cols = x.shape
    _mat(residual, "residual")
    if residual.shape != x.shape:
        raise ValueError("residual must have the shape of x")
    _vec(gamma, cols, "gamma")
    _vec(beta, cols, "beta")
    y = _out_like(y, x, "y")
    h_ptr = None
    if h_out is not None:
        _out_like(h_out, x, "h_out")
        h_ptr = h_out.data_ptr()
    st = _capi.lib().residual_layernorm_f32_ws(x.data_ptr(), residual.data_ptr(), gamma.data_ptr(),
                                                beta.data_ptr(), y.data_ptr(), h_ptr, rows, cols,
                                                float(eps), _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("residual_layernorm_f32", st)
    return y


def cross_entropy_f32(logits, targets, loss=None, plan=None, workspace=None, stream=None):
    """loss[r] = logsumexp_c logits[r,c] - logits[r, targets[r]]. Returns loss."""
    torch = _torch()
    _mat(logits, "logits")
    rows, cols = logits.shape
    _vec(targets, rows, "targets", dtype=torch.int32)
    loss = _out_rows(loss, logits, "loss")
    st = _capi.lib().cross_entropy_f32_ws(logits.data_ptr(), targets.data_ptr(), loss.data_ptr(),
                                           rows, cols, _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("cross_entropy_f32", st)
    return loss


# ---- bfloat16 storage: float arithmetic, one rounding per stored element -----

def _bf16():
    return _torch().bfloat16


def rmsnorm_bf16(x, w, eps=1e-6, y=None, plan=None, workspace=None, stream=None):
    """rmsnorm_f32 on bfloat16 x, w, y. Returns y."""
    _mat(x, "x", _bf16())
    rows, cols = x.shape
    _vec(w, cols, "w", _bf16())
    y = _out_like(y, x, "y")
    st = _capi.lib().rmsnorm_bf16_ws(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, cols, float(eps),
                                      _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("rmsnorm_bf16", st)
    return y


def row_sum_bf16(x, out=None, plan=None, workspace=None, stream=None):
    """Row sums of bfloat16 x as float32 (float64 accumulation). Returns out."""
    _mat(x, "x", _bf16())
    rows, cols = x.shape
    out = _out_rows(out, x, "out")
    st = _capi.lib().row_sum_bf16_ws(x.data_ptr(), out.data_ptr(), rows, cols, _plan_ptr(plan),
                                      *_ws(workspace), _stream(stream))
    _capi.check("row_sum_bf16", st)
    return out


def softmax_bf16(x, y=None, plan=None, workspace=None, stream=None):
    """softmax_f32 on bfloat16 x, y. Returns y."""
    _mat(x, "x", _bf16())
    rows, cols = x.shape
    y = _out_like(y, x, "y")
    st = _capi.lib().softmax_bf16_ws(x.data_ptr(), y.data_ptr(), rows, cols, _plan_ptr(plan),
                                      *_ws(workspace), _stream(stream))
    _capi.check("softmax_bf16", st)
    return y


def layernorm_bf16(x, gamma, beta, eps=1e-5, y=None, plan=None, workspace=None, stream=None):
    """layernorm_f32 on bfloat16 x, gamma, beta, y. Returns y."""
    _mat(x, "x", _bf16())
    rows, cols = x.shape
    _vec(gamma, cols, "gamma", _bf16())
    _vec(beta, cols, "beta", _bf16())
    y = _out_like(y, x, "y")
    st = _capi.lib().layernorm_bf16_ws(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), y.data_ptr(),
                                        rows, cols, float(eps), _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("layernorm_bf16", st)
    return y


def residual_layernorm_bf16(x, residual, gamma, beta, eps=1e-5, y=None, h_out=None, plan=None,
                            workspace=None, stream=None):
    """h = bf16(x + residual); y = LayerNorm(h), bfloat16 storage. Returns y."""
    _mat(x, "x", _bf16())
    rows, cols = x.shape
    _mat(residual, "residual", _bf16())
    if residual.shape != x.shape:
        raise ValueError("residual must have the shape of x")
    _vec(gamma, cols, "gamma", _bf16())
    _vec(beta, cols, "beta", _bf16())
    y = _out_like(y, x, "y")
    h_ptr = None
    if h_out is not None:
        _out_like(h_out, x, "h_out")
        h_ptr = h_out.data_ptr()
    st = _capi.lib().residual_layernorm_bf16_ws(x.data_ptr(), residual.data_ptr(), gamma.data_ptr(),
                                                 beta.data_ptr(), y.data_ptr(), h_ptr, rows, cols,
                                                 float(eps), _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("residual_layernorm_bf16", st)
    return y


def cross_entropy_bf16(logits, targets, loss=None, plan=None, workspace=None, stream=None):
    """cross_entropy_f32 on bfloat16 logits; float32 loss. Returns loss."""
    torch = _torch()
    _mat(logits, "logits", _bf16())
    rows, cols = logits.shape
    _vec(targets, rows, "targets", dtype=torch.int32)
    loss = _out_rows(loss, logits, "loss")
    st = _capi.lib().cross_entropy_bf16_ws(logits.data_ptr(), targets.data_ptr(), loss.data_ptr(),
                                            rows, cols, _plan_ptr(plan), *_ws(workspace), _stream(stream))
    _capi.check("cross_entropy_bf16", st)
    return loss


def rr_workspace_bytes(op, rows, cols, plan=None) -> int:
    """Workspace bytes `plan` needs on (rows, cols) (the selected plan when
    None, given unlimited workspace); 0 when it needs none."""
    op_id = OP_IDS[op] if isinstance(op, str) else int(op)
    n = _capi.lib().rr_workspace_bytes(op_id, rows, cols, _plan_ptr(plan))
    if n < 0:
        raise RowRedError("rr_workspace_bytes", _capi.RR_ERR_INVALID_ARGUMENT)
    return n


def rr_select_plan(op, rows, cols) -> rr_plan:
    """Plan the library picks for (op, rows, cols); op is a name or an rr_op value."""
    op_id = OP_IDS[op] if isinstance(op, str) else int(op)
    p = rr_plan()
    _capi.check("rr_select_plan", _capi.lib().rr_select_plan(op_id, rows, cols, p))
    return p


def batch_problem(op, x, w=None, beta=None, residual=None, targets=None, eps=None, y=None, h_out=None,
                  out=None):
    """One problem for rr_batch on torch tensors: `op` is an operator name
    ("rmsnorm", "layernorm_bf16", ...); w is RMSNorm's w or LayerNorm's
    gamma; outputs not given are allocated. Returns (rr_problem, outputs)
    where outputs maps "y", "h" or "out" to the tensors the call writes; the
    caller keeps every tensor alive until the batch has run."""
    torch = _torch()
    bf = op.endswith("_bf16")
    base = op[:-5] if bf else op
    if base not in ("rmsnorm", "sum", "softmax", "layernorm", "residual_layernorm", "cross_entropy"):
        raise ValueError(f"unknown operator {op!r}")
    dt = _bf16() if bf else torch.float32
    _mat(x, "x", dt)
    rows, cols = x.shape
    p = _capi.rr_problem()
    p.op, p.rows, p.cols, p.x = OP_IDS[op], rows, cols, x.data_ptr()
    outs = {}
    if base in ("rmsnorm", "layernorm", "residual_layernorm"):
        _vec(w, cols, "w", dt)
        p.w = w.data_ptr()
        p.eps = float(eps if eps is not None else (1e-6 if base == "rmsnorm" else 1e-5))
    if base in ("layernorm", "residual_layernorm"):
        _vec(beta, cols, "beta", dt)
        p.beta = beta.data_ptr()
    if base == "residual_layernorm":
        _mat(residual, "residual", dt)
        if residual.shape != x.shape:
            raise ValueError("residual must have the shape of x")
        p.residual = residual.data_ptr()
        if h_out is not None:
            outs["h"] = _out_like(h_out, x, "h_out")
            p.h_out = h_out.data_ptr()
    if base == "cross_entropy":
        if not isinstance(targets, torch.Tensor) or targets.dtype != torch.int32 or not targets.is_cuda \
                or targets.shape != (rows,) or not targets.is_contiguous():
            raise TypeError("targets must be a contiguous int32 CUDA/HIP tensor of shape (rows,)")
        p.targets = targets.data_ptr()
    if base in ("sum", "cross_entropy"):
        outs["out"] = _out_rows(out, x, "out")
        p.row_out = outs["out"].data_ptr()
    else:
        outs["y"] = _out_like(y, x, "y")
        p.y = outs["y"].data_ptr()
    return p, outs


def rr_batch(problems, stream=None) -> None:
    """Run up to RR_BATCH_MAX problems (from batch_problem) in one kernel launch."""
    arr = (_capi.rr_problem * max(1, len(problems)))(*problems)
    _capi.check("rr_batch", _capi.lib().rr_batch(arr, len(problems), _stream(stream)))


def rr_select_plan_from(op, rows, cols, source) -> rr_plan:
    """Plan of one source for (op, rows, cols): "auto", "table", "model" or
    "rule" (or an rr_plan_source value)."""
    src = {"auto": 0, "table": 1, "model": 2, "rule": 3}.get(source, source)
    op_id = OP_IDS[op] if isinstance(op, str) else int(op)
    p = rr_plan()
    _capi.check("rr_select_plan_from", _capi.lib().rr_select_plan_from(op_id, rows, cols, int(src), p))
    return p


def rr_model_time_us(op, rows, cols, plan) -> float:
    """The analytic model's predicted microseconds per launch of `plan`
    (-1.0 for an illegal or split plan)."""
    op_id = OP_IDS[op] if isinstance(op, str) else int(op)
    return _capi.lib().rr_model_time_us(op_id, rows, cols, _plan_ptr(plan))


def rr_check_plan(op, rows, cols, plan) -> int:
    """rr_status of the legality check of `plan` for (op, rows, cols)."""
    op_id = OP_IDS[op] if isinstance(op, str) else int(op)
    return _capi.lib().rr_check_plan(op_id, rows, cols, _plan_ptr(plan))


def rr_status_string(status: int) -> str:
    return _capi.status_string(status)


def rr_copy_f32(src, dst, stream=None):
    """dst[:] = src[:] through the library's streaming copy kernel."""
    torch = _torch()
    for t, n in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda \
                or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous float32 CUDA/HIP tensor")
    if src.numel() != dst.numel():
        raise ValueError("src and dst sizes differ")
    _capi.check("rr_copy_f32", _capi.lib().rr_copy_f32(src.data_ptr(), dst.data_ptr(), src.numel(),
                                                        _stream(stream)))
    return dst


def rr_stream_f32(src, dst, copy=True, packs_per_thread=1, block=256, stream=None):
    """Streaming kernel of a chosen geometry over src (float32): copy into dst,
    or (copy=False) read only, dst being passed but never written. dst needs
    src's size for a copy, else at least one float per thread launched."""
    torch = _torch()
    for t, n in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda \
                or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous float32 CUDA/HIP tensor")
    n = src.numel()
    need = n if copy else -(-n // (4 * packs_per_thread * block)) * block
    if dst.numel() < need:
        raise ValueError(f"dst holds {dst.numel()} floats, {need} needed")
    _capi.check("rr_stream_f32", _capi.lib().rr_stream_f32(src.data_ptr(), dst.data_ptr(), n, int(bool(copy)),
                                                            packs_per_thread, block, _stream(stream)))
    return dst


def rr_empty_kernel(stream=None):
    _capi.check("rr_empty_kernel", _capi.lib().rr_empty_kernel(_stream(stream)))

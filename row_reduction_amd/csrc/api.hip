// C entry points of librowred: argument validation, plan selection or check,
// and the kernel launch(es) on the caller's stream. No allocation, no
// synchronisation, no global mutable state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "internal.h"

namespace rowred {
namespace {

bool aligned(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

// A required pointer: present and aligned to its element size.
bool ok_ptr(const void *p, uintptr_t bytes) { return p != nullptr && aligned(p, bytes); }
// An optional pointer: null, or aligned to its element size.
bool ok_opt(const void *p, uintptr_t bytes) { return p == nullptr || aligned(p, bytes); }

bool ok_eps(float eps) { return isfinite(eps) && eps >= 0.0f; }

int check_shape(int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return RR_ERR_INVALID_ARGUMENT;
    if (cols > 0x7fffffff) return RR_ERR_UNSUPPORTED;
    return RR_OK;
}

// Widest bfloat16 pack (2V bytes, V <= 8) that the alignment of every given
// pointer allows; null pointers impose nothing.
int max_v_for(std::initializer_list<const void *> ptrs) {
    uintptr_t bits = 0;
    for (const void *p : ptrs) bits |= reinterpret_cast<uintptr_t>(p);
    int v = 8;
    while (v > 1 && (bits & (uintptr_t)(2 * v - 1))) v /= 2;
    return v;
}

bool bf16_op(int op) { return op >= RR_OP_RMSNORM_BF16; }

int launch(int op, const rr_plan &p, const Args &a, void *stream) {
    switch (op) {
        case RR_OP_RMSNORM: return launch_rmsnorm(p, a, stream);
        case RR_OP_SUM: return launch_row_sum(p, a, stream);
        case RR_OP_SOFTMAX: return launch_softmax(p, a, stream);
        case RR_OP_LAYERNORM: return launch_layernorm(p, a, stream);
        case RR_OP_RESIDUAL_LAYERNORM: return launch_residual_layernorm(p, a, stream);
        case RR_OP_CROSS_ENTROPY: return launch_cross_entropy(p, a, stream);
        case RR_OP_RMSNORM_BF16: return launch_rmsnorm_bf16(p, a, stream);
        case RR_OP_SUM_BF16: return launch_row_sum_bf16(p, a, stream);
        case RR_OP_SOFTMAX_BF16: return launch_softmax_bf16(p, a, stream);
        case RR_OP_LAYERNORM_BF16: return launch_layernorm_bf16(p, a, stream);
        case RR_OP_RESIDUAL_LAYERNORM_BF16: return launch_residual_layernorm_bf16(p, a, stream);
        case RR_OP_CROSS_ENTROPY_BF16: return launch_cross_entropy_bf16(p, a, stream);
        default: return (int)hipErrorInvalidValue;
    }
}

// Everything after pointer validation: workspace check, plan (the caller's,
// checked, or the selector's within max_v and the workspace), launch.
// max_v bounds the pack width by the pointers' alignment (bfloat16 storage).
int run(int op, Args a, const rr_plan *plan, void *workspace, int64_t workspace_bytes, int max_v,
        void *stream) {
    if (workspace_bytes < 0 || !ok_opt(workspace, 16)) return RR_ERR_INVALID_ARGUMENT;
    const int64_t avail = workspace != nullptr ? workspace_bytes : 0;
    rr_plan p;
    if (plan != nullptr) {
        int st = check_plan(op, a.rows, a.cols, plan);
        if (st != RR_OK) return st == RR_ERR_INVALID_ARGUMENT ? RR_ERR_INVALID_ARGUMENT : RR_ERR_UNSUPPORTED;
        if (plan->v > max_v) return RR_ERR_UNSUPPORTED;
        if (plan_workspace_bytes(a.rows, a.cols, plan) > avail) return RR_ERR_UNSUPPORTED;
        p = *plan;
    } else {
        int st = select_plan(op, a.rows, a.cols, &p, max_v, avail);
        if (st != RR_OK) return st;
    }
    a.workspace = workspace;
    return launch(op, p, a, stream) == (int)hipSuccess ? RR_OK : RR_ERR_LAUNCH;
}

Args base_args(int64_t rows, int64_t cols) {
    Args a = {};
    a.rows = rows;
    a.cols = (int32_t)cols;
    return a;
}

// Per-operator front ends shared by the float and bfloat16 entry points;
// E is the element size of the row and weight tensors.
int rmsnorm_call(int op, uintptr_t E, const void *x, const void *w, void *y, int64_t rows, int64_t cols,
                 float eps, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x, E) || !ok_ptr(w, E) || !ok_ptr(y, E) || !ok_eps(eps)) return RR_ERR_INVALID_ARGUMENT;
    Args a = base_args(rows, cols);
    a.x = x;
    a.w = w;
    a.y = y;
    a.eps = eps;
    return run(op, a, plan, ws, wsb, bf16_op(op) ? max_v_for({x, w, y}) : 8, stream);
}

int row_sum_call(int op, uintptr_t E, const void *x, float *out, int64_t rows, int64_t cols,
                 const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x, E) || !ok_ptr(out, 4)) return RR_ERR_INVALID_ARGUMENT;
    Args a = base_args(rows, cols);
    a.x = x;
    a.row_out = out;
    return run(op, a, plan, ws, wsb, bf16_op(op) ? max_v_for({x}) : 8, stream);
}

int softmax_call(int op, uintptr_t E, const void *x, void *y, int64_t rows, int64_t cols,
                 const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x, E) || !ok_ptr(y, E)) return RR_ERR_INVALID_ARGUMENT;
    Args a = base_args(rows, cols);
    a.x = x;
    a.y = y;
    return run(op, a, plan, ws, wsb, bf16_op(op) ? max_v_for({x, y}) : 8, stream);
}

int layernorm_call(int op, uintptr_t E, const void *x, const void *residual, const void *gamma,
                   const void *beta, void *y, void *h_out, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    const bool residual_op = (op == RR_OP_RESIDUAL_LAYERNORM || op == RR_OP_RESIDUAL_LAYERNORM_BF16);
    if (!ok_ptr(x, E) || !ok_ptr(gamma, E) || !ok_ptr(beta, E) || !ok_ptr(y, E) || !ok_eps(eps) ||
        (residual_op && !ok_ptr(residual, E)) || !ok_opt(h_out, E))
        return RR_ERR_INVALID_ARGUMENT;
    Args a = base_args(rows, cols);
    a.x = x;
    a.residual = residual;
    a.w = gamma;
    a.beta = beta;
    a.y = y;
    a.h_out = h_out;
    a.eps = eps;
    return run(op, a, plan, ws, wsb, bf16_op(op) ? max_v_for({x, residual, gamma, beta, y, h_out}) : 8,
               stream);
}

int cross_entropy_call(int op, uintptr_t E, const void *logits, const int32_t *targets, float *loss,
                       int64_t rows, int64_t cols, const rr_plan *plan, void *ws, int64_t wsb,
                       void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(logits, E) || !ok_ptr(targets, 4) || !ok_ptr(loss, 4)) return RR_ERR_INVALID_ARGUMENT;
    Args a = base_args(rows, cols);
    a.x = logits;
    a.targets = targets;
    a.row_out = loss;
    return run(op, a, plan, ws, wsb, bf16_op(op) ? max_v_for({logits}) : 8, stream);
}

}  // namespace
}  // namespace rowred

using namespace rowred;

extern "C" {

// ---- float storage ---------------------------------------------------------------

int rmsnorm_f32_ws(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return rmsnorm_call(RR_OP_RMSNORM, 4, x, w, y, rows, cols, eps, plan, ws, wsb, stream);
}
int rmsnorm_f32_ex(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *stream) {
    return rmsnorm_f32_ws(x, w, y, rows, cols, eps, plan, nullptr, 0, stream);
}
int rmsnorm_f32(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                void *stream) {
    return rmsnorm_f32_ws(x, w, y, rows, cols, eps, nullptr, nullptr, 0, stream);
}

int row_sum_f32_ws(const float *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan, void *ws,
                   int64_t wsb, void *stream) {
    return row_sum_call(RR_OP_SUM, 4, x, out, rows, cols, plan, ws, wsb, stream);
}
int row_sum_f32_ex(const float *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                   void *stream) {
    return row_sum_f32_ws(x, out, rows, cols, plan, nullptr, 0, stream);
}
int row_sum_f32(const float *x, float *out, int64_t rows, int64_t cols, void *stream) {
    return row_sum_f32_ws(x, out, rows, cols, nullptr, nullptr, 0, stream);
}

int softmax_f32_ws(const float *x, float *y, int64_t rows, int64_t cols, const rr_plan *plan, void *ws,
                   int64_t wsb, void *stream) {
    return softmax_call(RR_OP_SOFTMAX, 4, x, y, rows, cols, plan, ws, wsb, stream);
}
int softmax_f32_ex(const float *x, float *y, int64_t rows, int64_t cols, const rr_plan *plan,
                   void *stream) {
    return softmax_f32_ws(x, y, rows, cols, plan, nullptr, 0, stream);
}
int softmax_f32(const float *x, float *y, int64_t rows, int64_t cols, void *stream) {
    return softmax_f32_ws(x, y, rows, cols, nullptr, nullptr, 0, stream);
}

int layernorm_f32_ws(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                     int64_t cols, float eps, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return layernorm_call(RR_OP_LAYERNORM, 4, x, nullptr, gamma, beta, y, nullptr, rows, cols, eps, plan,
                          ws, wsb, stream);
}
int layernorm_f32_ex(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                     int64_t cols, float eps, const rr_plan *plan, void *stream) {
    return layernorm_f32_ws(x, gamma, beta, y, rows, cols, eps, plan, nullptr, 0, stream);
}
int layernorm_f32(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                  int64_t cols, float eps, void *stream) {
    return layernorm_f32_ws(x, gamma, beta, y, rows, cols, eps, nullptr, nullptr, 0, stream);
}

int residual_layernorm_f32_ws(const float *x, const float *residual, const float *gamma,
                              const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                              float eps, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return layernorm_call(RR_OP_RESIDUAL_LAYERNORM, 4, x, residual, gamma, beta, y, h_out, rows, cols, eps,
                          plan, ws, wsb, stream);
}
int residual_layernorm_f32_ex(const float *x, const float *residual, const float *gamma,
                              const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                              float eps, const rr_plan *plan, void *stream) {
    return residual_layernorm_f32_ws(x, residual, gamma, beta, y, h_out, rows, cols, eps, plan, nullptr, 0,
                                     stream);
}
int residual_layernorm_f32(const float *x, const float *residual, const float *gamma,
                           const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                           float eps, void *stream) {
    return residual_layernorm_f32_ws(x, residual, gamma, beta, y, h_out, rows, cols, eps, nullptr, nullptr,
                                     0, stream);
}

int cross_entropy_f32_ws(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                         int64_t cols, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return cross_entropy_call(RR_OP_CROSS_ENTROPY, 4, logits, targets, loss, rows, cols, plan, ws, wsb,
                              stream);
}
int cross_entropy_f32_ex(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                         int64_t cols, const rr_plan *plan, void *stream) {
    return cross_entropy_f32_ws(logits, targets, loss, rows, cols, plan, nullptr, 0, stream);
}
int cross_entropy_f32(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                      int64_t cols, void *stream) {
    return cross_entropy_f32_ws(logits, targets, loss, rows, cols, nullptr, nullptr, 0, stream);
}

// ---- bfloat16 storage ------------------------------------------------------------

int rmsnorm_bf16_ws(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                    float eps, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return rmsnorm_call(RR_OP_RMSNORM_BF16, 2, x, w, y, rows, cols, eps, plan, ws, wsb, stream);
}
int rmsnorm_bf16_ex(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                    float eps, const rr_plan *plan, void *stream) {
    return rmsnorm_bf16_ws(x, w, y, rows, cols, eps, plan, nullptr, 0, stream);
}
int rmsnorm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                 float eps, void *stream) {
    return rmsnorm_bf16_ws(x, w, y, rows, cols, eps, nullptr, nullptr, 0, stream);
}

int row_sum_bf16_ws(const uint16_t *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *ws, int64_t wsb, void *stream) {
    return row_sum_call(RR_OP_SUM_BF16, 2, x, out, rows, cols, plan, ws, wsb, stream);
}
int row_sum_bf16_ex(const uint16_t *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *stream) {
    return row_sum_bf16_ws(x, out, rows, cols, plan, nullptr, 0, stream);
}
int row_sum_bf16(const uint16_t *x, float *out, int64_t rows, int64_t cols, void *stream) {
    return row_sum_bf16_ws(x, out, rows, cols, nullptr, nullptr, 0, stream);
}

int softmax_bf16_ws(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *ws, int64_t wsb, void *stream) {
    return softmax_call(RR_OP_SOFTMAX_BF16, 2, x, y, rows, cols, plan, ws, wsb, stream);
}
int softmax_bf16_ex(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *stream) {
    return softmax_bf16_ws(x, y, rows, cols, plan, nullptr, 0, stream);
}
int softmax_bf16(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, void *stream) {
    return softmax_bf16_ws(x, y, rows, cols, nullptr, nullptr, 0, stream);
}

int layernorm_bf16_ws(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                      int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *ws, int64_t wsb,
                      void *stream) {
    return layernorm_call(RR_OP_LAYERNORM_BF16, 2, x, nullptr, gamma, beta, y, nullptr, rows, cols, eps,
                          plan, ws, wsb, stream);
}
int layernorm_bf16_ex(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                      int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream) {
    return layernorm_bf16_ws(x, gamma, beta, y, rows, cols, eps, plan, nullptr, 0, stream);
}
int layernorm_bf16(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                   int64_t rows, int64_t cols, float eps, void *stream) {
    return layernorm_bf16_ws(x, gamma, beta, y, rows, cols, eps, nullptr, nullptr, 0, stream);
}

int residual_layernorm_bf16_ws(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                               const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                               int64_t cols, float eps, const rr_plan *plan, void *ws, int64_t wsb,
                               void *stream) {
    return layernorm_call(RR_OP_RESIDUAL_LAYERNORM_BF16, 2, x, residual, gamma, beta, y, h_out, rows, cols,
                          eps, plan, ws, wsb, stream);
}
int residual_layernorm_bf16_ex(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                               const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                               int64_t cols, float eps, const rr_plan *plan, void *stream) {
    return residual_layernorm_bf16_ws(x, residual, gamma, beta, y, h_out, rows, cols, eps, plan, nullptr,
                                      0, stream);
}
int residual_layernorm_bf16(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                            const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                            int64_t cols, float eps, void *stream) {
    return residual_layernorm_bf16_ws(x, residual, gamma, beta, y, h_out, rows, cols, eps, nullptr,
                                      nullptr, 0, stream);
}

int cross_entropy_bf16_ws(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                          int64_t cols, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return cross_entropy_call(RR_OP_CROSS_ENTROPY_BF16, 2, logits, targets, loss, rows, cols, plan, ws,
                              wsb, stream);
}
int cross_entropy_bf16_ex(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                          int64_t cols, const rr_plan *plan, void *stream) {
    return cross_entropy_bf16_ws(logits, targets, loss, rows, cols, plan, nullptr, 0, stream);
}
int cross_entropy_bf16(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                       int64_t cols, void *stream) {
    return cross_entropy_bf16_ws(logits, targets, loss, rows, cols, nullptr, nullptr, 0, stream);
}

// ---- planner ---------------------------------------------------------------------

int rr_select_plan(int op, int64_t rows, int64_t cols, rr_plan *out) {
    return select_plan(op, rows, cols, out);
}

int rr_check_plan(int op, int64_t rows, int64_t cols, const rr_plan *plan) {
    return check_plan(op, rows, cols, plan);
}

int rr_select_plan_from(int op, int64_t rows, int64_t cols, int source, rr_plan *out) {
    return select_plan_from(op, rows, cols, source, out);
}

double rr_model_time_us(int op, int64_t rows, int64_t cols, const rr_plan *plan) {
    return model_time_us(op, rows, cols, plan);
}

int64_t rr_workspace_bytes(int op, int64_t rows, int64_t cols, const rr_plan *plan) {
    rr_plan p;
    if (plan != nullptr) {
        if (check_plan(op, rows, cols, plan) != RR_OK) return -1;
        p = *plan;
    } else if (select_plan(op, rows, cols, &p, 8, INT64_MAX) != RR_OK) {
        return -1;
    }
    return plan_workspace_bytes(rows, cols, &p);
}

const char *rr_status_string(int status) {
    switch (status) {
        case RR_OK: return "RR_OK";
        case RR_ERR_INVALID_ARGUMENT: return "RR_ERR_INVALID_ARGUMENT";
        case RR_ERR_UNSUPPORTED: return "RR_ERR_UNSUPPORTED";
        case RR_ERR_LAUNCH: return "RR_ERR_LAUNCH";
        default: return "RR_UNKNOWN_STATUS";
    }
}

}  // extern "C"

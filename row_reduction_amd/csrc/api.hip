// C entry points of librowred: argument validation, plan selection or check,
// and one kernel launch on the caller's stream. No allocation, no
// synchronisation, no global mutable state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "internal.h"

namespace rowred {
namespace {

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A required pointer: present and dword aligned.
bool ok_ptr(const void *p) { return p != nullptr && aligned4(p); }

bool ok_eps(float eps) { return isfinite(eps) && eps >= 0.0f; }

int check_shape(int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return RR_ERR_INVALID_ARGUMENT;
    if (cols > 0x7fffffff) return RR_ERR_UNSUPPORTED;
    return RR_OK;
}

// A required bfloat16 pointer: present and 2-byte aligned.
bool ok_ptr16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

// Widest bfloat16 pack (2V bytes, V <= 8) that the alignment of every given
// pointer allows; null pointers impose nothing.
int max_v_for(std::initializer_list<const void *> ptrs) {
    uintptr_t bits = 0;
    for (const void *p : ptrs) bits |= reinterpret_cast<uintptr_t>(p);
    int v = 8;
    while (v > 1 && (bits & (uintptr_t)(2 * v - 1))) v /= 2;
    return v;
}

// Plan for the call: the caller's (checked) or the selector's. max_v bounds
// the pack width by the pointers' alignment (bfloat16 storage).
int resolve_plan(int op, int64_t rows, int64_t cols, const rr_plan *plan, rr_plan *out, int max_v = 8) {
    if (plan != nullptr) {
        int st = check_plan(op, rows, cols, plan);
        if (st != RR_OK) return st == RR_ERR_INVALID_ARGUMENT ? RR_ERR_INVALID_ARGUMENT : RR_ERR_UNSUPPORTED;
        if (plan->v > max_v) return RR_ERR_UNSUPPORTED;
        *out = *plan;
        return RR_OK;
    }
    return select_plan(op, rows, cols, out, max_v);
}

Args base_args(int64_t rows, int64_t cols) {
    Args a = {};
    a.rows = rows;
    a.cols = (int32_t)cols;
    return a;
}

int finish(int hip_status) { return hip_status == (int)hipSuccess ? RR_OK : RR_ERR_LAUNCH; }

}  // namespace
}  // namespace rowred

using namespace rowred;

extern "C" {

int rmsnorm_f32_ex(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x) || !ok_ptr(w) || !ok_ptr(y) || !ok_eps(eps)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_RMSNORM, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.w = w;
    a.y = y;
    a.eps = eps;
    return finish(launch_rmsnorm(p, a, stream));
}

int rmsnorm_f32(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                void *stream) {
    return rmsnorm_f32_ex(x, w, y, rows, cols, eps, nullptr, stream);
}

int row_sum_f32_ex(const float *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                   void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x) || !ok_ptr(out)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_SUM, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.row_out = out;
    return finish(launch_row_sum(p, a, stream));
}

int row_sum_f32(const float *x, float *out, int64_t rows, int64_t cols, void *stream) {
    return row_sum_f32_ex(x, out, rows, cols, nullptr, stream);
}

int softmax_f32_ex(const float *x, float *y, int64_t rows, int64_t cols, const rr_plan *plan,
                   void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x) || !ok_ptr(y)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_SOFTMAX, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.y = y;
    return finish(launch_softmax(p, a, stream));
}

int softmax_f32(const float *x, float *y, int64_t rows, int64_t cols, void *stream) {
    return softmax_f32_ex(x, y, rows, cols, nullptr, stream);
}

int layernorm_f32_ex(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                     int64_t cols, float eps, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x) || !ok_ptr(gamma) || !ok_ptr(beta) || !ok_ptr(y) || !ok_eps(eps))
        return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_LAYERNORM, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.w = gamma;
    a.beta = beta;
    a.y = y;
    a.eps = eps;
    return finish(launch_layernorm(p, a, stream));
}

int layernorm_f32(const float *x, const float *gamma, const float *beta, float *y, int64_t rows,
                  int64_t cols, float eps, void *stream) {
    return layernorm_f32_ex(x, gamma, beta, y, rows, cols, eps, nullptr, stream);
}

int residual_layernorm_f32_ex(const float *x, const float *residual, const float *gamma,
                              const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                              float eps, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(x) || !ok_ptr(residual) || !ok_ptr(gamma) || !ok_ptr(beta) || !ok_ptr(y) ||
        !ok_eps(eps) || (h_out != nullptr && !aligned4(h_out)))
        return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_RESIDUAL_LAYERNORM, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.residual = residual;
    a.w = gamma;
    a.beta = beta;
    a.y = y;
    a.h_out = h_out;
    a.eps = eps;
    return finish(launch_residual_layernorm(p, a, stream));
}

int residual_layernorm_f32(const float *x, const float *residual, const float *gamma,
                           const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                           float eps, void *stream) {
    return residual_layernorm_f32_ex(x, residual, gamma, beta, y, h_out, rows, cols, eps, nullptr,
                                     stream);
}

int cross_entropy_f32_ex(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                         int64_t cols, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr(logits) || !ok_ptr(targets) || !ok_ptr(loss)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_CROSS_ENTROPY, rows, cols, plan, &p)) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = logits;
    a.targets = targets;
    a.row_out = loss;
    return finish(launch_cross_entropy(p, a, stream));
}

int cross_entropy_f32(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                      int64_t cols, void *stream) {
    return cross_entropy_f32_ex(logits, targets, loss, rows, cols, nullptr, stream);
}

// ---- bfloat16 storage -----------------------------------------------------------

int rmsnorm_bf16_ex(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                    float eps, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(x) || !ok_ptr16(w) || !ok_ptr16(y) || !ok_eps(eps)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_RMSNORM_BF16, rows, cols, plan, &p, max_v_for({x, w, y}))) != RR_OK)
        return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.w = w;
    a.y = y;
    a.eps = eps;
    return finish(launch_rmsnorm_bf16(p, a, stream));
}

int rmsnorm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                 float eps, void *stream) {
    return rmsnorm_bf16_ex(x, w, y, rows, cols, eps, nullptr, stream);
}

int row_sum_bf16_ex(const uint16_t *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(x) || !ok_ptr(out)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_SUM_BF16, rows, cols, plan, &p, max_v_for({x}))) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.row_out = out;
    return finish(launch_row_sum_bf16(p, a, stream));
}

int row_sum_bf16(const uint16_t *x, float *out, int64_t rows, int64_t cols, void *stream) {
    return row_sum_bf16_ex(x, out, rows, cols, nullptr, stream);
}

int softmax_bf16_ex(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, const rr_plan *plan,
                    void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(x) || !ok_ptr16(y)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_SOFTMAX_BF16, rows, cols, plan, &p, max_v_for({x, y}))) != RR_OK) return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.y = y;
    return finish(launch_softmax_bf16(p, a, stream));
}

int softmax_bf16(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, void *stream) {
    return softmax_bf16_ex(x, y, rows, cols, nullptr, stream);
}

int layernorm_bf16_ex(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                      int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(x) || !ok_ptr16(gamma) || !ok_ptr16(beta) || !ok_ptr16(y) || !ok_eps(eps))
        return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_LAYERNORM_BF16, rows, cols, plan, &p, max_v_for({x, gamma, beta, y}))) != RR_OK)
        return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.w = gamma;
    a.beta = beta;
    a.y = y;
    a.eps = eps;
    return finish(launch_layernorm_bf16(p, a, stream));
}

int layernorm_bf16(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                   int64_t rows, int64_t cols, float eps, void *stream) {
    return layernorm_bf16_ex(x, gamma, beta, y, rows, cols, eps, nullptr, stream);
}

int residual_layernorm_bf16_ex(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                               const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                               int64_t cols, float eps, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(x) || !ok_ptr16(residual) || !ok_ptr16(gamma) || !ok_ptr16(beta) || !ok_ptr16(y) ||
        !ok_eps(eps) || (h_out != nullptr && !ok_ptr16(h_out)))
        return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_RESIDUAL_LAYERNORM_BF16, rows, cols, plan, &p,
                           max_v_for({x, residual, gamma, beta, y, h_out}))) != RR_OK)
        return st;
    Args a = base_args(rows, cols);
    a.x = x;
    a.residual = residual;
    a.w = gamma;
    a.beta = beta;
    a.y = y;
    a.h_out = h_out;
    a.eps = eps;
    return finish(launch_residual_layernorm_bf16(p, a, stream));
}

int residual_layernorm_bf16(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                            const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                            int64_t cols, float eps, void *stream) {
    return residual_layernorm_bf16_ex(x, residual, gamma, beta, y, h_out, rows, cols, eps, nullptr,
                                      stream);
}

int cross_entropy_bf16_ex(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                          int64_t cols, const rr_plan *plan, void *stream) {
    int st = check_shape(rows, cols);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!ok_ptr16(logits) || !ok_ptr(targets) || !ok_ptr(loss)) return RR_ERR_INVALID_ARGUMENT;
    rr_plan p;
    if ((st = resolve_plan(RR_OP_CROSS_ENTROPY_BF16, rows, cols, plan, &p, max_v_for({logits}))) != RR_OK)
        return st;
    Args a = base_args(rows, cols);
    a.x = logits;
    a.targets = targets;
    a.row_out = loss;
    return finish(launch_cross_entropy_bf16(p, a, stream));
}

int cross_entropy_bf16(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                       int64_t cols, void *stream) {
    return cross_entropy_bf16_ex(logits, targets, loss, rows, cols, nullptr, stream);
}

int rr_select_plan(int op, int64_t rows, int64_t cols, rr_plan *out) {
    return select_plan(op, rows, cols, out);
}

int rr_check_plan(int op, int64_t rows, int64_t cols, const rr_plan *plan) {
    return check_plan(op, rows, cols, plan);
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

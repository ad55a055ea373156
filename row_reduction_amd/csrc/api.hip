// C entry points of librowred: argument validation, plan selection or check,
// and the kernel launch(es) on the caller's stream. No allocation, no
// synchronisation, and no state shared between calls other than the static
// device buffer of rmsnorm_f32_noalloc (with its per-device address).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "batch.h"
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
    if (cols > RR_MAX_COLS) return RR_ERR_UNSUPPORTED;
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

// The plan a call runs: the caller's, checked (its pack width within max_v,
// its workspace within `avail` bytes), or the selector's within both.
int resolve_plan(int op, const Args &a, const rr_plan *plan, int64_t avail, int max_v, rr_plan *out) {
    if (plan != nullptr) {
        int st = check_plan(op, a.rows, a.cols, plan);
        if (st != RR_OK) return st == RR_ERR_INVALID_ARGUMENT ? RR_ERR_INVALID_ARGUMENT : RR_ERR_UNSUPPORTED;
        if (plan->v > max_v) return RR_ERR_UNSUPPORTED;
        if (plan_workspace_bytes(a.rows, a.cols, plan) > avail) return RR_ERR_UNSUPPORTED;
        *out = *plan;
        return RR_OK;
    }
    return select_plan(op, a.rows, a.cols, out, max_v, avail);
}

// Everything after pointer validation: workspace check, plan (the caller's,
// checked, or the selector's within max_v and the workspace), launch.
// max_v bounds the pack width by the pointers' alignment (bfloat16 storage).
int run(int op, Args a, const rr_plan *plan, void *workspace, int64_t workspace_bytes, int max_v,
        void *stream) {
    if (workspace_bytes < 0 || !ok_opt(workspace, 16)) return RR_ERR_INVALID_ARGUMENT;
    const int64_t avail = workspace != nullptr ? workspace_bytes : 0;
    rr_plan p;
    const int st = resolve_plan(op, a, plan, avail, max_v, &p);
    if (st != RR_OK) return st;
    a.workspace = workspace;
    return launch(op, p, a, stream) == (int)hipSuccess ? RR_OK : RR_ERR_LAUNCH;
}

Args base_args(int64_t rows, int64_t cols) {
    Args a = {};
    a.rows = rows;
    a.cols = (int32_t)cols;
    return a;
}

// The operands of one operator call, as the entry points and rr_batch get them.
struct Operands {
    const void *x = nullptr, *residual = nullptr, *w = nullptr, *beta = nullptr;
    const int32_t *targets = nullptr;
    void *y = nullptr, *h_out = nullptr;
    float *row_out = nullptr;
    int64_t rows = 0, cols = 0;
    float eps = 0.0f;
};

// Validation shared by every entry point and rr_batch: shape first; with
// rows == 0 nothing is read or written and the pointers are not looked at;
// else every required pointer present and aligned to its element size (E =
// 2 for bfloat16 rows and weights, 4 for float; int32 targets and float
// per-row outputs 4), optional ones null or aligned, eps finite and >= 0.
// Fills the kernel arguments and the widest bfloat16 pack the pointers'
// alignment allows.
int prepare(int op, const Operands &o, Args *a, int *max_v) {
    const int st = check_shape(o.rows, o.cols);
    if (st != RR_OK) return st;
    *a = base_args(o.rows, o.cols);
    *max_v = 8;
    if (o.rows == 0) return RR_OK;
    const bool bf = bf16_op(op);
    const uintptr_t E = bf ? 2 : 4;
    switch (bf ? op - RR_OP_RMSNORM_BF16 : op) {
        case RR_OP_RMSNORM:
            if (!ok_ptr(o.x, E) || !ok_ptr(o.w, E) || !ok_ptr(o.y, E) || !ok_eps(o.eps))
                return RR_ERR_INVALID_ARGUMENT;
            if (bf) *max_v = max_v_for({o.x, o.w, o.y});
            break;
        case RR_OP_SUM:
            if (!ok_ptr(o.x, E) || !ok_ptr(o.row_out, 4)) return RR_ERR_INVALID_ARGUMENT;
            if (bf) *max_v = max_v_for({o.x});
            break;
        case RR_OP_SOFTMAX:
            if (!ok_ptr(o.x, E) || !ok_ptr(o.y, E)) return RR_ERR_INVALID_ARGUMENT;
            if (bf) *max_v = max_v_for({o.x, o.y});
            break;
        case RR_OP_LAYERNORM:
        case RR_OP_RESIDUAL_LAYERNORM: {
            const bool residual_op = (op == RR_OP_RESIDUAL_LAYERNORM || op == RR_OP_RESIDUAL_LAYERNORM_BF16);
            if (!ok_ptr(o.x, E) || !ok_ptr(o.w, E) || !ok_ptr(o.beta, E) || !ok_ptr(o.y, E) ||
                !ok_eps(o.eps) || (residual_op && !ok_ptr(o.residual, E)) || !ok_opt(o.h_out, E))
                return RR_ERR_INVALID_ARGUMENT;
            if (bf) *max_v = max_v_for({o.x, o.residual, o.w, o.beta, o.y, o.h_out});
            break;
        }
        case RR_OP_CROSS_ENTROPY:
            if (!ok_ptr(o.x, E) || !ok_ptr(o.targets, 4) || !ok_ptr(o.row_out, 4))
                return RR_ERR_INVALID_ARGUMENT;
            if (bf) *max_v = max_v_for({o.x});
            break;
        default:
            return RR_ERR_INVALID_ARGUMENT;
    }
    // Only the operands the operator uses reach the kernel.
    const int base = bf ? op - RR_OP_RMSNORM_BF16 : op;
    a->x = o.x;
    if (base == RR_OP_RESIDUAL_LAYERNORM) a->residual = o.residual;
    if (base == RR_OP_RMSNORM || base == RR_OP_LAYERNORM || base == RR_OP_RESIDUAL_LAYERNORM) a->w = o.w;
    if (base == RR_OP_LAYERNORM || base == RR_OP_RESIDUAL_LAYERNORM) a->beta = o.beta;
    if (base == RR_OP_CROSS_ENTROPY) a->targets = o.targets;
    if (base != RR_OP_SUM && base != RR_OP_CROSS_ENTROPY) a->y = o.y;
    if (base == RR_OP_RESIDUAL_LAYERNORM) a->h_out = o.h_out;
    if (base == RR_OP_SUM || base == RR_OP_CROSS_ENTROPY) a->row_out = o.row_out;
    if (base == RR_OP_RMSNORM || base == RR_OP_LAYERNORM || base == RR_OP_RESIDUAL_LAYERNORM) a->eps = o.eps;
    return RR_OK;
}

int call_op(int op, const Operands &o, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    Args a;
    int max_v;
    const int st = prepare(op, o, &a, &max_v);
    if (st != RR_OK || o.rows == 0) return st;
    return run(op, a, plan, ws, wsb, max_v, stream);
}

// Per-operator front ends shared by the float and bfloat16 entry points.
int rmsnorm_call(int op, const void *x, const void *w, void *y, int64_t rows, int64_t cols, float eps,
                 const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    Operands o;
    o.x = x;
    o.w = w;
    o.y = y;
    o.rows = rows;
    o.cols = cols;
    o.eps = eps;
    return call_op(op, o, plan, ws, wsb, stream);
}

int row_sum_call(int op, const void *x, float *out, int64_t rows, int64_t cols, const rr_plan *plan,
                 void *ws, int64_t wsb, void *stream) {
    Operands o;
    o.x = x;
    o.row_out = out;
    o.rows = rows;
    o.cols = cols;
    return call_op(op, o, plan, ws, wsb, stream);
}

int softmax_call(int op, const void *x, void *y, int64_t rows, int64_t cols, const rr_plan *plan, void *ws,
                 int64_t wsb, void *stream) {
    Operands o;
    o.x = x;
    o.y = y;
    o.rows = rows;
    o.cols = cols;
    return call_op(op, o, plan, ws, wsb, stream);
}

int layernorm_call(int op, const void *x, const void *residual, const void *gamma, const void *beta, void *y,
                   void *h_out, int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *ws,
                   int64_t wsb, void *stream) {
    Operands o;
    o.x = x;
    o.residual = residual;
    o.w = gamma;
    o.beta = beta;
    o.y = y;
    o.h_out = h_out;
    o.rows = rows;
    o.cols = cols;
    o.eps = eps;
    return call_op(op, o, plan, ws, wsb, stream);
}

int cross_entropy_call(int op, const void *logits, const int32_t *targets, float *loss, int64_t rows,
                       int64_t cols, const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    Operands o;
    o.x = logits;
    o.targets = targets;
    o.row_out = loss;
    o.rows = rows;
    o.cols = cols;
    return call_op(op, o, plan, ws, wsb, stream);
}

}  // namespace
}  // namespace rowred

using namespace rowred;

extern "C" {

// ---- float storage ---------------------------------------------------------------

int rmsnorm_f32_ws(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *ws, int64_t wsb, void *stream) {
    return rmsnorm_call(RR_OP_RMSNORM, x, w, y, rows, cols, eps, plan, ws, wsb, stream);
}
int rmsnorm_f32_noalloc(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                        const rr_plan *plan, void *stream) {
    Operands o;
    o.x = x;
    o.w = w;
    o.y = y;
    o.rows = rows;
    o.cols = cols;
    o.eps = eps;
    Args a;
    int max_v;
    int st = prepare(RR_OP_RMSNORM, o, &a, &max_v);
    if (st != RR_OK || rows == 0) return st;
    rr_plan p;
    st = resolve_plan(RR_OP_RMSNORM, a, plan, RR_NOALLOC_SCRATCH_BYTES, max_v, &p);
    if (st != RR_OK) return st;
    if (p.path == RR_PATH_SPLIT) {
        st = noalloc_scratch(stream, &a.workspace);
        if (st != RR_OK) return st;
    }
    return launch(RR_OP_RMSNORM, p, a, stream) == (int)hipSuccess ? RR_OK : RR_ERR_LAUNCH;
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
    return row_sum_call(RR_OP_SUM, x, out, rows, cols, plan, ws, wsb, stream);
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
    return softmax_call(RR_OP_SOFTMAX, x, y, rows, cols, plan, ws, wsb, stream);
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
    return layernorm_call(RR_OP_LAYERNORM, x, nullptr, gamma, beta, y, nullptr, rows, cols, eps, plan,
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
    return layernorm_call(RR_OP_RESIDUAL_LAYERNORM, x, residual, gamma, beta, y, h_out, rows, cols, eps,
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
    return cross_entropy_call(RR_OP_CROSS_ENTROPY, logits, targets, loss, rows, cols, plan, ws, wsb,
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
    return rmsnorm_call(RR_OP_RMSNORM_BF16, x, w, y, rows, cols, eps, plan, ws, wsb, stream);
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
    return row_sum_call(RR_OP_SUM_BF16, x, out, rows, cols, plan, ws, wsb, stream);
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
    return softmax_call(RR_OP_SOFTMAX_BF16, x, y, rows, cols, plan, ws, wsb, stream);
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
    return layernorm_call(RR_OP_LAYERNORM_BF16, x, nullptr, gamma, beta, y, nullptr, rows, cols, eps,
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
    return layernorm_call(RR_OP_RESIDUAL_LAYERNORM_BF16, x, residual, gamma, beta, y, h_out, rows, cols,
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
    return cross_entropy_call(RR_OP_CROSS_ENTROPY_BF16, logits, targets, loss, rows, cols, plan, ws,
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

int rr_batch(const rr_problem *problems, int32_t count, void *stream) {
    if (count < 0 || count > RR_BATCH_MAX || (count > 0 && problems == nullptr)) return RR_ERR_INVALID_ARGUMENT;
    BatchArgs b = {};
    int n = 0;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const rr_problem &q = problems[i];
        Operands o;
        o.x = q.x;
        o.residual = q.residual;
        o.w = q.w;
        o.beta = q.beta;
        o.targets = q.targets;
        o.y = q.y;
        o.h_out = q.h_out;
        o.row_out = q.row_out;
        o.rows = q.rows;
        o.cols = q.cols;
        o.eps = q.eps;
        Args a;
        int max_v;
        const int st = prepare(q.op, o, &a, &max_v);
        if (st != RR_OK) return st;
        if (q.rows == 0) continue;
        const bool wide = bf16_op(q.op) ? (max_v >= 8 && q.cols % 8 == 0) : q.cols >= 4;
        BatchProblem &p = b.p[n++];
        p.x = a.x;
        p.residual = a.residual;
        p.w = a.w;
        p.beta = a.beta;
        p.targets = a.targets;
        p.y = a.y;
        p.h_out = a.h_out;
        p.row_out = a.row_out;
        p.rows = a.rows;
        p.first_block = blocks;
        p.cols = a.cols;
        p.variant = 2 * q.op + (wide ? 1 : 0);
        p.eps = a.eps;
        // A whole group per row from 2048 columns up, else a wavefront per row.
        p.lanes = a.cols >= 2048 ? 256 : 64;
        const int64_t per_group = 256 / p.lanes;
        blocks += (a.rows + per_group - 1) / per_group;
    }
    if (blocks > 0x7fffffff) return RR_ERR_UNSUPPORTED;
    if (n == 0) return RR_OK;
    b.count = n;
    return launch_batch(b, blocks, stream) == (int)hipSuccess ? RR_OK : RR_ERR_LAUNCH;
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

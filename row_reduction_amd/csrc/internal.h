// Shared between the host entry points and the device kernels of librowred.
#pragma once

#include <stdint.h>

#include "rowred.h"

namespace rowred {

// Everything one launch needs, passed by value as the kernel argument.
// Row and weight tensors are float or bfloat16 (the kernel instance decides);
// per-row outputs are always float.
struct Args {
    const void *x;           // input rows (logits for cross-entropy)
    const void *residual;    // residual LayerNorm second input, else null
    const void *w;           // RMSNorm weight / LayerNorm gamma, else null
    const void *beta;        // LayerNorm beta, else null
    const int32_t *targets;  // cross-entropy targets, else null
    void *y;                 // per-element output, else null
    void *h_out;             // residual LayerNorm h = x + residual, may be null
    float *row_out;          // per-row output (row sum, loss), else null
    void *workspace;         // split rows: rows x slices partials (16 bytes each), else null
    int64_t rows;
    int32_t cols;
    int32_t lanes_per_row;   // workers per row (power of two)
    int32_t log2_lanes;      // log2(lanes_per_row)
    int32_t rows_per_group;  // rows handled by one workgroup
    float eps;
};

// Host-side launchers, one translation unit per operator. Each validates
// nothing (the entry points do) and returns the HIP status of the launch.
int launch_rmsnorm(const rr_plan &p, const Args &a, void *stream);
int launch_row_sum(const rr_plan &p, const Args &a, void *stream);
int launch_softmax(const rr_plan &p, const Args &a, void *stream);
int launch_layernorm(const rr_plan &p, const Args &a, void *stream);
int launch_residual_layernorm(const rr_plan &p, const Args &a, void *stream);
int launch_cross_entropy(const rr_plan &p, const Args &a, void *stream);
int launch_rmsnorm_bf16(const rr_plan &p, const Args &a, void *stream);
int launch_row_sum_bf16(const rr_plan &p, const Args &a, void *stream);
int launch_softmax_bf16(const rr_plan &p, const Args &a, void *stream);
int launch_layernorm_bf16(const rr_plan &p, const Args &a, void *stream);
int launch_residual_layernorm_bf16(const rr_plan &p, const Args &a, void *stream);
int launch_cross_entropy_bf16(const rr_plan &p, const Args &a, void *stream);

// Device address, on the device `stream` belongs to (the calling thread's
// current device for the null stream), of the static buffer
// rmsnorm_f32_noalloc keeps its split-row partials in
// (RR_NOALLOC_SCRATCH_BYTES); looked up once per device. RR_OK, or
// RR_ERR_INVALID_ARGUMENT (the stream's device cannot be queried),
// RR_ERR_UNSUPPORTED / RR_ERR_LAUNCH when no address can be had.
int noalloc_scratch(void *stream, void **out);

// Planner (plan.cpp; pure host C++).
// max_v: widest pack the caller's pointer alignment allows (bfloat16 ops);
// workspace_bytes > 0 lets the selector pick a split plan that fits in it.
int select_plan(int op, int64_t rows, int64_t cols, rr_plan *out, int max_v = 8,
                int64_t workspace_bytes = 0);
int check_plan(int op, int64_t rows, int64_t cols, const rr_plan *plan);
// Workspace a (legal) plan needs: rows x slices x 16 bytes for split plans, else 0.
int64_t plan_workspace_bytes(int64_t rows, int64_t cols, const rr_plan *plan);
// Plan from one source (rr_plan_source); the analytic model's predicted time.
int select_plan_from(int op, int64_t rows, int64_t cols, int source, rr_plan *out);
double model_time_us(int op, int64_t rows, int64_t cols, const rr_plan *plan);

}  // namespace rowred

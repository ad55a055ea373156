// Batched launch: several independent problems of any operators in one
// kernel. Each 256-thread workgroup serves the problem whose group range
// holds blockIdx.x, running the streaming row body (a single pass for the
// statistics, a second for the outputs where the operator has per-element
// outputs) either on four of its rows, one wavefront each, or on one row with
// all four wavefronts. Wavefronts past the problem's last row exit: with one
// wavefront per row the body has no barrier.
#include "batch.h"
#include "device.h"

namespace rowred {
namespace {

__global__ void __launch_bounds__(256) batch_kernel(const BatchArgs b) {
    const int64_t blk = blockIdx.x;
    int i = 0;
    while (i + 1 < b.count && b.p[i + 1].first_block <= blk) ++i;
    const BatchProblem &q = b.p[i];
    Args a = {};
    a.x = q.x;
    a.residual = q.residual;
    a.w = q.w;
    a.beta = q.beta;
    a.targets = q.targets;
    a.y = q.y;
    a.h_out = q.h_out;
    a.row_out = q.row_out;
    a.rows = q.rows;
    a.cols = q.cols;
    a.lanes_per_row = q.lanes;
    a.log2_lanes = q.lanes == 256 ? 8 : 6;
    a.rows_per_group = 256 / q.lanes;
    a.eps = q.eps;
    const int64_t row = (blk - q.first_block) * a.rows_per_group + (threadIdx.x >> a.log2_lanes);
    if (row >= q.rows) return;  // only when lanes == 64: a whole wavefront, no barrier follows
    switch (q.variant) {
#define ROWRED_BATCH_CASES(OPID, KOP, WIDE, T)                            \
    case 2 * (OPID): loop_row<KOP, 1, 0, 0, 0, T>(a, row); break;            \
    case 2 * (OPID) + 1: loop_row<KOP, WIDE, 0, 0, 0, T>(a, row); break;
        ROWRED_BATCH_CASES(RR_OP_RMSNORM, kRmsNorm, 4, float)
        ROWRED_BATCH_CASES(RR_OP_SUM, kSum, 4, float)
        ROWRED_BATCH_CASES(RR_OP_SOFTMAX, kSoftmax, 4, float)
        ROWRED_BATCH_CASES(RR_OP_LAYERNORM, kLayerNorm, 4, float)
        ROWRED_BATCH_CASES(RR_OP_RESIDUAL_LAYERNORM, kResidualLayerNorm, 4, float)
        ROWRED_BATCH_CASES(RR_OP_CROSS_ENTROPY, kCrossEntropy, 4, float)
        ROWRED_BATCH_CASES(RR_OP_RMSNORM_BF16, kRmsNorm, 8, bf16_t)
        ROWRED_BATCH_CASES(RR_OP_SUM_BF16, kSum, 8, bf16_t)
        ROWRED_BATCH_CASES(RR_OP_SOFTMAX_BF16, kSoftmax, 8, bf16_t)
        ROWRED_BATCH_CASES(RR_OP_LAYERNORM_BF16, kLayerNorm, 8, bf16_t)
        ROWRED_BATCH_CASES(RR_OP_RESIDUAL_LAYERNORM_BF16, kResidualLayerNorm, 8, bf16_t)
        ROWRED_BATCH_CASES(RR_OP_CROSS_ENTROPY_BF16, kCrossEntropy, 8, bf16_t)
#undef ROWRED_BATCH_CASES
        default: break;
    }
}

}  // namespace

int launch_batch(const BatchArgs &b, int64_t blocks, void *stream) {
    hipLaunchKernelGGL(batch_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), b);
    return (int)hipGetLastError();
}

}  // namespace rowred

// Shared between the host entry point rr_batch and its kernel.
#pragma once

#include <stdint.h>

#include "rowred.h"

namespace rowred {

// Batched launch (rr_batch): up to kBatchMax problems in one kernel of
// 256-thread groups on the streaming row body; problem i owns the groups
// [first_block, first_block + ceil(rows / (256 / lanes))), each holding
// 256 / lanes of its rows (lanes = 64 or 256 per row).
constexpr int kBatchMax = RR_BATCH_MAX;
struct BatchProblem {
    const void *x, *residual, *w, *beta;
    const int32_t *targets;
    void *y, *h_out;
    float *row_out;
    int64_t rows;
    int64_t first_block;
    int32_t cols;
    int32_t variant;  // 2 * rr_op + 1 when the row takes the wide pack (float 4, bfloat16 8)
    float eps;
    int32_t lanes;    // lanes per row: 64 (four rows per group) or 256 (one)
};
struct BatchArgs {
    BatchProblem p[kBatchMax];
    int32_t count;
};
static_assert(sizeof(BatchArgs) <= 3584, "batched kernel arguments stay well inside the 4 KiB limit");
int launch_batch(const BatchArgs &b, int64_t blocks, void *stream);

}  // namespace rowred

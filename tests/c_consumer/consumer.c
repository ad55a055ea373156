/* A plain C99 consumer of the C ABI: includes only rowred.h, links
 * librowred.so, and uses the host-side calls (plan selection, legality,
 * workspace sizing, status strings, argument validation); no GPU needed. */
#include <stdio.h>
#include <string.h>

#include "rowred.h"

static int fail(const char *what) {
    fprintf(stderr, "FAIL: %s\n", what);
    return 1;
}

int main(void) {
    rr_plan p;
    if (rr_select_plan(RR_OP_RMSNORM, 16384, 8192, &p) != RR_OK) return fail("select");
    if (rr_check_plan(RR_OP_RMSNORM, 16384, 8192, &p) != RR_OK) return fail("check selected");
    if (p.rows_per_group * p.lanes_per_row != p.block) return fail("rows_per_group * lanes");
    if (rr_select_plan(RR_OP_SOFTMAX_BF16, 2048, 128256, &p) != RR_OK) return fail("select bf16");
    if (rr_select_plan_from(RR_OP_LAYERNORM, 300, 777, RR_PLAN_MODEL, &p) != RR_OK) return fail("model");
    if (!(rr_model_time_us(RR_OP_LAYERNORM, 300, 777, &p) > 0.0)) return fail("model time");
    if (rr_workspace_bytes(RR_OP_SUM, 1, 1 << 20, NULL) <= 0) return fail("split workspace");
    if (rr_workspace_bytes(RR_OP_SUM, 4096, 4096, NULL) != 0) return fail("no workspace");
    if (strcmp(rr_status_string(RR_ERR_UNSUPPORTED), "RR_ERR_UNSUPPORTED") != 0) return fail("status");
    /* Validation before any launch: bad shapes and arguments are refused. */
    if (rmsnorm_f32(NULL, NULL, NULL, -1, 8, 1e-6f, NULL) != RR_ERR_INVALID_ARGUMENT) return fail("rows < 0");
    if (rmsnorm_f32(NULL, NULL, NULL, 0, 8, 1e-6f, NULL) != RR_OK) return fail("rows == 0");
    if (softmax_f32(NULL, NULL, 4, 8, NULL) != RR_ERR_INVALID_ARGUMENT) return fail("null x");
    if (rr_batch(NULL, 0, NULL) != RR_OK) return fail("empty batch");
    printf("ok\n");
    return 0;
}

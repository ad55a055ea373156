/*
 * rowred.h — FP32 row reductions for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Every operator reduces each row of a row-major, contiguous float32 matrix
 * x[rows][cols] independently. Sources of the definitions:
 *   - RMSNorm and its calling convention (input, weight, output, eps; rows*cols
 *     inputs and outputs, cols weights; 0 < cols; FP32 reduction and epilogue
 *     with rounding only on the output store): meTile, "Thread Ownership and
 *     Software Staging", section "Register-tiled reductions" (the register
 *     RMSNorm kernel's contract).
 *   - The sibling operators (row sum, softmax, LayerNorm, residual LayerNorm,
 *     cross-entropy) on one reduction core: LuisaCompute notes, "Consecutive-
 *     worker reduction layout checkpoint", section "Evidence and what remains"
 *     (the operator-coverage item). Their formulas are the textbook ones and
 *     are stated on each declaration below.
 *   - The worker / V ownership map behind rr_plan: same LuisaCompute page,
 *     section "Implementation and semantics".
 *   - Fail-closed geometry (an illegal plan is rejected, never remapped):
 *     meTile page above, section "Compiler-selected communication" (the
 *     thread-limit check), and the LuisaCompute page, section "Verification
 *     checkpoint" (invalid widths and resource overflow fail closed).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (hipMalloc / PyTorch CUDA tensors) owned by
 *     the caller; all tensors are contiguous row-major float32 (targets int32),
 *     at least 4-byte aligned. Outputs are preallocated by the caller.
 *   - The library allocates nothing, frees nothing and never synchronises: it
 *     enqueues one kernel (two for a split plan) on `stream` (a hipStream_t;
 *     NULL = the default stream) and returns. Faults during execution surface at the caller's
 *     next synchronisation.
 *   - y may alias x exactly (in-place); any other overlap between an output
 *     and an input is undefined.
 *   - Return value is an rr_status. rows == 0 returns RR_OK without touching
 *     the GPU. rows < 0, cols <= 0, a NULL required pointer (when rows > 0), a
 *     pointer not 4-byte aligned, or an eps that is negative or not finite
 *     return RR_ERR_INVALID_ARGUMENT. cols > RR_MAX_COLS, a grid beyond the device
 *     limit, or an explicit plan that is illegal for (op, rows, cols) return
 *     RR_ERR_UNSUPPORTED. A launch the HIP runtime refuses returns
 *     RR_ERR_LAUNCH. Nothing is enqueued unless RR_OK is returned.
 *   - All entry points are reentrant and may be called concurrently from
 *     several host threads. No state is shared between calls (each host
 *     thread keeps its own small cache of the plan model's recent choices),
 *     except the static device buffer of rmsnorm_f32_noalloc, whose calls
 *     on one GPU must not overlap.
 *   - Arithmetic is float32 (row sum: float64 accumulation, see below); the
 *     order of additions inside a row depends on the plan, as the ownership
 *     map permits.
 */
#ifndef ROWRED_H
#define ROWRED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rr_status {
    RR_OK = 0,
    RR_ERR_INVALID_ARGUMENT = 1,
    RR_ERR_UNSUPPORTED = 2,
    RR_ERR_LAUNCH = 3
} rr_status;

typedef enum rr_op {
    RR_OP_RMSNORM = 0,
    RR_OP_SUM = 1,
    RR_OP_SOFTMAX = 2,
    RR_OP_LAYERNORM = 3,
    RR_OP_RESIDUAL_LAYERNORM = 4,
    RR_OP_CROSS_ENTROPY = 5,
    /* The same operators with bfloat16 storage (see the *_bf16 entry points). */
    RR_OP_RMSNORM_BF16 = 6,
    RR_OP_SUM_BF16 = 7,
    RR_OP_SOFTMAX_BF16 = 8,
    RR_OP_LAYERNORM_BF16 = 9,
    RR_OP_RESIDUAL_LAYERNORM_BF16 = 10,
    RR_OP_CROSS_ENTROPY_BF16 = 11
} rr_op;

/* How rows map onto workgroups.
 *   RR_PATH_PACKED: lanes_per_row < 64 — several rows share one 64-lane
 *                   wavefront; each row is reduced inside its lane segment.
 *   RR_PATH_ROW:    lanes_per_row >= 64 — one row spans lanes_per_row/64 whole
 *                   wavefronts (combined through LDS with one barrier per
 *                   reduction); a workgroup may hold several rows.
 *   RR_PATH_LOOP:   one row per workgroup, any cols: statistics in one pass
 *                   over the row, then (RMSNorm, softmax, LayerNorm,
 *                   residual LayerNorm) a second pass that re-reads the
 *                   values not kept in registers or LDS.
 *   RR_PATH_SPLIT:  a row is cut into S = ceil(cols / (lanes_per_row * slots))
 *                   slices, one workgroup each (2 <= S <= 1024, rows <= 65535):
 *                   a first launch keeps each slice in registers and writes
 *                   one 16-byte partial per (row, slice) to a caller-provided
 *                   workspace, a second merges the partials in slice order
 *                   and writes the outputs (re-reading the slice for the
 *                   per-element operators). Only through the *_ws entry
 *                   points; v = 4 (float) or 8 (bfloat16, cols % 8 == 0),
 *                   slots 16 or 32, cache 2. */
/* Widest row accepted: 2^31 - 2^20 columns, so that every column index a
 * kernel forms (a pack start plus up to one chunk or slice span) fits in 32
 * bits. */
#define RR_MAX_COLS (((int64_t)1 << 31) - ((int64_t)1 << 20))

typedef enum rr_path {
    RR_PATH_PACKED = 0,
    RR_PATH_ROW = 1,
    RR_PATH_LOOP = 2,
    RR_PATH_SPLIT = 3
} rr_path;

/* A launch plan. Worker w (0 <= w < lanes_per_row) of a row owns logical
 * columns i = (chunk * lanes_per_row + w) * v + e for 0 <= e < v, and keeps
 * them in private slot chunk * v + e (LuisaCompute page, section
 * "Implementation and semantics").
 *   path            rr_path
 *   block           threads per workgroup: 64, 128, 256, 512 or 1024
 *   lanes_per_row   workers per row: power of two, 8..1024, <= block
 *                   (LOOP: equal to block)
 *   rows_per_group  block / lanes_per_row (LOOP: 1)
 *   v               consecutive elements per worker pack: 1, 2 or 4 for
 *                   float rows; 1, 2, 4 or 8 for bfloat16 rows, where v > 1
 *                   also needs cols % v == 0 and every tensor pointer
 *                   aligned to 2*v bytes (one naturally aligned access per
 *                   pack, at most 16 bytes)
 *   slots           values each worker keeps in registers: chunks * v with
 *                   chunks in {1, 2, 4, 8} and slots <= 32;
 *                   cols <= lanes_per_row * slots. On the LOOP path the
 *                   values kept in registers between the two passes: 0;
 *                   32 for the two-pass operators with v >= 4; with
 *                   v >= 4 and 1024-lane groups also 64 (RMSNorm, softmax)
 *                   and 96 (softmax). 1024-lane softmax plans keeping 64
 *                   or 96, and LayerNorm plans keeping 32, hold 32 more
 *                   values per lane in LDS; for bfloat16 rows LayerNorm
 *                   and residual LayerNorm at 32 and softmax at 64 hold 72
 *                   there instead (as bfloat16), and so does RMSNorm at 64
 *                   with v = 8.
 *   cache           cache policy for the row data: 0 = default; 1 = output
 *                   stores non-temporal; 2 = row loads (x, residual) and
 *                   output stores non-temporal (on the LOOP path only the
 *                   last pass's loads). Weights (w, gamma, beta) are
 *                   always loaded with the default policy. Results do not
 *                   depend on it. */
typedef struct rr_plan {
    int32_t path;
    int32_t block;
    int32_t lanes_per_row;
    int32_t rows_per_group;
    int32_t v;
    int32_t slots;
    int32_t cache;
} rr_plan;

/* RMSNorm: y[r,c] = x[r,c] * w[c] / sqrt(mean_c x[r,c]^2 + eps).
 * x, y: rows*cols floats; w: cols floats. */
int rmsnorm_f32(const float *x, const float *w, float *y,
                int64_t rows, int64_t cols, float eps, void *stream);

/* Row sum: out[r] = sum_c x[r,c]. Accumulates in float64 and rounds once,
 * so the result is within float32 rounding of the exact sum even when
 * positive and negative terms cancel. out: rows floats. */
int row_sum_f32(const float *x, float *out, int64_t rows, int64_t cols, void *stream);

/* Softmax with the row maximum subtracted:
 * y[r,c] = exp(x[r,c] - m_r) / sum_k exp(x[r,k] - m_r), m_r = max_k x[r,k].
 * -inf entries (masked positions) get 0; a row of -inf only gives NaN, as
 * the definition does (-inf - -inf). */
int softmax_f32(const float *x, float *y, int64_t rows, int64_t cols, void *stream);

/* LayerNorm: y = (x - mean_r) / sqrt(var_r + eps) * gamma[c] + beta[c], with
 * the population variance var_r = mean_c (x[r,c] - mean_r)^2. Rows held in
 * registers take corrected two-pass statistics; longer rows take one pass
 * that merges per-pack statistics of the values shifted by the row's first
 * value, so rows whose variance is tiny next to mean^2 stay accurate either
 * way. gamma, beta: cols floats. */
int layernorm_f32(const float *x, const float *gamma, const float *beta, float *y,
                  int64_t rows, int64_t cols, float eps, void *stream);

/* Residual LayerNorm: h = x + residual rounded to float32, then LayerNorm of h.
 * h_out may be NULL; otherwise it receives h (rows*cols floats, bit-exact
 * float32 sums). */
int residual_layernorm_f32(const float *x, const float *residual,
                           const float *gamma, const float *beta,
                           float *y, float *h_out,
                           int64_t rows, int64_t cols, float eps, void *stream);

/* Cross-entropy per row with int32 class targets:
 * loss[r] = log sum_c exp(x[r,c] - m_r) + m_r - x[r, targets[r]].
 * -inf logits add nothing to the sum; a -inf target logit gives +inf.
 * Targets are not validated on the host (that would need a synchronisation):
 * a target outside [0, cols) yields loss = NaN and no out-of-bounds read.
 * targets, loss: rows elements. */
int cross_entropy_f32(const float *logits, const int32_t *targets, float *loss,
                      int64_t rows, int64_t cols, void *stream);

/* Explicit-plan forms. plan == NULL selects the plan as the plain forms do;
 * otherwise the plan must be legal for (op, rows, cols) — checked exactly as
 * rr_check_plan does — or RR_ERR_UNSUPPORTED is returned. */
int rmsnorm_f32_ex(const float *x, const float *w, float *y,
                   int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream);
int row_sum_f32_ex(const float *x, float *out, int64_t rows, int64_t cols,
                   const rr_plan *plan, void *stream);
int softmax_f32_ex(const float *x, float *y, int64_t rows, int64_t cols,
                   const rr_plan *plan, void *stream);
int layernorm_f32_ex(const float *x, const float *gamma, const float *beta, float *y,
                     int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream);
int residual_layernorm_f32_ex(const float *x, const float *residual,
                              const float *gamma, const float *beta,
                              float *y, float *h_out, int64_t rows, int64_t cols, float eps,
                              const rr_plan *plan, void *stream);
int cross_entropy_f32_ex(const float *logits, const int32_t *targets, float *loss,
                         int64_t rows, int64_t cols, const rr_plan *plan, void *stream);

/* ---- bfloat16 storage ------------------------------------------------------
 * The same six operators on bfloat16 tensors, passed as uint16_t bit
 * patterns: inputs are widened exactly to float, every reduction and the
 * epilogue run in float (row sum in float64), and each element output is
 * rounded to bfloat16 (nearest, ties to even) once, on the store — the
 * 16-bit-I/O, FP32-arithmetic form the meTile page measures (section
 * "Measurements and reproduction"). Weights (w, gamma, beta) are bfloat16 too;
 * per-row outputs (row sum, loss) are float. Tensor pointers must be at least
 * 2-byte aligned (else RR_ERR_INVALID_ARGUMENT); the selected plan uses the
 * widest pack the pointers' alignment allows, and an explicit plan whose v
 * needs more alignment than the pointers have returns RR_ERR_UNSUPPORTED.
 * Residual LayerNorm rounds h = x + residual to bfloat16 before normalising
 * (h materialised at the tensors' precision) and stores that h in h_out. */
int rmsnorm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y,
                 int64_t rows, int64_t cols, float eps, void *stream);
int row_sum_bf16(const uint16_t *x, float *out, int64_t rows, int64_t cols, void *stream);
int softmax_bf16(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols, void *stream);
int layernorm_bf16(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                   int64_t rows, int64_t cols, float eps, void *stream);
int residual_layernorm_bf16(const uint16_t *x, const uint16_t *residual,
                            const uint16_t *gamma, const uint16_t *beta,
                            uint16_t *y, uint16_t *h_out,
                            int64_t rows, int64_t cols, float eps, void *stream);
int cross_entropy_bf16(const uint16_t *logits, const int32_t *targets, float *loss,
                       int64_t rows, int64_t cols, void *stream);
int rmsnorm_bf16_ex(const uint16_t *x, const uint16_t *w, uint16_t *y,
                    int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream);
int row_sum_bf16_ex(const uint16_t *x, float *out, int64_t rows, int64_t cols,
                    const rr_plan *plan, void *stream);
int softmax_bf16_ex(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols,
                    const rr_plan *plan, void *stream);
int layernorm_bf16_ex(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                      int64_t rows, int64_t cols, float eps, const rr_plan *plan, void *stream);
int residual_layernorm_bf16_ex(const uint16_t *x, const uint16_t *residual,
                               const uint16_t *gamma, const uint16_t *beta,
                               uint16_t *y, uint16_t *h_out, int64_t rows, int64_t cols, float eps,
                               const rr_plan *plan, void *stream);
int cross_entropy_bf16_ex(const uint16_t *logits, const int32_t *targets, float *loss,
                          int64_t rows, int64_t cols, const rr_plan *plan, void *stream);

/* ---- split rows with a caller workspace --------------------------------------
 * The *_ws forms take, besides an optional explicit plan, a device workspace
 * of workspace_bytes bytes (16-byte aligned, caller-owned; its contents need
 * no initialisation and are scratch between the two launches of a split
 * plan). With plan == NULL the selector may then pick RR_PATH_SPLIT for
 * shapes with few (under 256), long rows when workspace_bytes suffices and
 * its measured per-operator cost model predicts the split faster than the
 * plain plan, else it picks as the plain forms do; an explicit split plan with too small a workspace
 * returns RR_ERR_UNSUPPORTED. Calls that share one workspace on different
 * streams race. rr_workspace_bytes gives the size a plan needs (the selected
 * one when plan == NULL): rows * S * 16 for a split plan, 0 otherwise, or
 * -1 for invalid arguments. These entry points exist for long rows that
 * leave most compute units idle on the one-workgroup-per-row paths (the
 * spreading of one long row across workers that the LuisaCompute page's
 * "Evidence and what remains" section names as next work). */
int64_t rr_workspace_bytes(int op, int64_t rows, int64_t cols, const rr_plan *plan);
int rmsnorm_f32_ws(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                   const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int row_sum_f32_ws(const float *x, float *out, int64_t rows, int64_t cols,
                   const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int softmax_f32_ws(const float *x, float *y, int64_t rows, int64_t cols,
                   const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int layernorm_f32_ws(const float *x, const float *gamma, const float *beta, float *y,
                     int64_t rows, int64_t cols, float eps,
                     const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int residual_layernorm_f32_ws(const float *x, const float *residual, const float *gamma,
                              const float *beta, float *y, float *h_out, int64_t rows, int64_t cols,
                              float eps, const rr_plan *plan, void *workspace,
                              int64_t workspace_bytes, void *stream);
int cross_entropy_f32_ws(const float *logits, const int32_t *targets, float *loss,
                         int64_t rows, int64_t cols,
                         const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int rmsnorm_bf16_ws(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                    float eps, const rr_plan *plan, void *workspace, int64_t workspace_bytes,
                    void *stream);
int row_sum_bf16_ws(const uint16_t *x, float *out, int64_t rows, int64_t cols,
                    const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int softmax_bf16_ws(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols,
                    const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int layernorm_bf16_ws(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                      int64_t rows, int64_t cols, float eps,
                      const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);
int residual_layernorm_bf16_ws(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                               const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                               int64_t cols, float eps, const rr_plan *plan, void *workspace,
                               int64_t workspace_bytes, void *stream);
int cross_entropy_bf16_ws(const uint16_t *logits, const int32_t *targets, float *loss,
                          int64_t rows, int64_t cols,
                          const rr_plan *plan, void *workspace, int64_t workspace_bytes, void *stream);

/* ---- split rows without any allocation ---------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc. As
 * rmsnorm_f32_ws, with the library's own static device buffer of
 * RR_NOALLOC_SCRATCH_BYTES (1 MiB: 65536 split partials) as the workspace;
 * the call allocates and frees nothing, directly or through any library.
 * With plan == NULL the selector may split rows whose partials fit the
 * buffer (rows * S * 16 bytes), else it picks as rmsnorm_f32 does; an
 * explicit split plan needing more returns RR_ERR_UNSUPPORTED before
 * anything is enqueued. Each GPU holds one such buffer, shared by every call
 * on that GPU, from the first call until the process ends; the copy used is
 * that of the device `stream` belongs to (for the null stream, the calling
 * thread's current device), its address looked up once per device
 * (RR_ERR_INVALID_ARGUMENT when the stream's device cannot be queried).
 * Nothing in it needs clearing (the first launch of a split plan writes
 * every partial the second one reads), but calls that overlap on one GPU
 * (other streams, other host threads) race on it: serialise them, e.g. on
 * one stream. Other arguments, ownership and
 * errors are as for rmsnorm_f32_ws (RR_ERR_LAUNCH also when the buffer's
 * device address cannot be obtained). */
#define RR_NOALLOC_SCRATCH_BYTES ((int64_t)1 << 20)
int rmsnorm_f32_noalloc(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps,
                        const rr_plan *plan, void *stream);

/* ---- Batched launch -------------------------------------------------------
 * Many small independent problems in one kernel launch, so that a sequence
 * of tiny operator calls pays one launch instead of one each (the per-launch
 * cost dominates below about 100 KB per call). Meant for small problems:
 * rows run the streaming row body (one pass for statistics, one for
 * outputs) on one 64-lane wavefront each, or on a whole 256-lane workgroup
 * from 2048 columns up, which is slower than the operator's own entry point
 * for large problems. */

#define RR_BATCH_MAX 32

/* One problem of a batch: op is an rr_op (float or bfloat16 storage); the
 * pointers mean what they mean in that operator's entry point (x = logits
 * for cross-entropy, w = gamma for the LayerNorms, row_out = row sum `out`
 * or cross-entropy `loss`); fields the operator does not use are ignored. */
typedef struct rr_problem {
    int32_t op;
    float eps;
    int64_t rows;
    int64_t cols;
    const void *x;
    const void *residual;
    const void *w;
    const void *beta;
    const int32_t *targets;
    void *y;
    void *h_out;
    float *row_out;
} rr_problem;

/* Runs problems[0 .. count-1] (0 <= count <= RR_BATCH_MAX) with one kernel
 * launch on `stream`; each problem's results equal its operator's (to the
 * same tolerance against the exact values; the reduction order differs).
 * Every problem is validated as its entry point would validate it before
 * anything is launched: any invalid problem fails the whole batch with that
 * entry point's status. Problems with rows == 0 are skipped; more than
 * 2^31-1 rows in total give RR_ERR_UNSUPPORTED. Problems must not write to
 * memory another problem of the batch reads or writes (they run
 * concurrently). The problems array is read during the call only. */
int rr_batch(const rr_problem *problems, int32_t count, void *stream);

/* Plan the library would use for (op, rows, cols): the measured per-shape
 * table entry when one exists, else the analytic model's cheapest legal
 * candidate (see rr_model_time_us). Pure host function; no GPU needed.
 * Returns RR_ERR_INVALID_ARGUMENT for an unknown op, rows < 0, cols <= 0 or
 * out == NULL, RR_ERR_UNSUPPORTED for cols > RR_MAX_COLS. The selected plan is
 * the one the plain entry points launch for suitably aligned pointers (the
 * *_ws forms with a large enough workspace may split few long rows instead). */
int rr_select_plan(int op, int64_t rows, int64_t cols, rr_plan *out);

/* Where a plan comes from (rr_select_plan_from).
 *   RR_PLAN_AUTO   what rr_select_plan returns
 *   RR_PLAN_TABLE  the frozen table of measured winners (RR_ERR_UNSUPPORTED
 *                  when the shape is not listed)
 *   RR_PLAN_MODEL  the analytic model's cheapest legal candidate
 *   RR_PLAN_RULE   the built-in rule the model replaced (kept for comparison) */
typedef enum rr_plan_source {
    RR_PLAN_AUTO = 0,
    RR_PLAN_TABLE = 1,
    RR_PLAN_MODEL = 2,
    RR_PLAN_RULE = 3
} rr_plan_source;

/* The plan of one source for (op, rows, cols), for full-alignment pointers.
 * Errors as rr_select_plan, plus RR_ERR_INVALID_ARGUMENT for an unknown
 * source. Pure host. */
int rr_select_plan_from(int op, int64_t rows, int64_t cols, int source, rr_plan *out);

/* Analytic cost model: predicted microseconds per launch of a legal
 * single-launch plan (PACKED, ROW or LOOP) on an MI355X (gfx950, 256 CUs),
 * launch floor included; -1.0 for an illegal plan, a split plan, or bad
 * arguments. Terms (after the LuisaCompute notes, "Consecutive-worker
 * reduction layout checkpoint", section "Evidence and what remains", which
 * ask for active groups and pack-width behaviour to be priced, and the MPP
 * memory notes' occupancy term): algorithmic bytes over a rate bounded by
 * HBM and by the bytes resident lanes keep in flight; rounds of resident
 * workgroups times a per-group latency chain; total lane-instructions; wave
 * and workgroup dispatch. Constants are fitted to the plan search's timings
 * (row_reduction_amd/data/plan_timings.csv). Meant for ranking plans of one
 * shape; absolute values are approximate. Pure host. */
double rr_model_time_us(int op, int64_t rows, int64_t cols, const rr_plan *plan);

/* RR_OK if `plan` is legal for (op, rows, cols), else RR_ERR_UNSUPPORTED
 * (RR_ERR_INVALID_ARGUMENT for bad op / shape / NULL plan). Pure host. */
int rr_check_plan(int op, int64_t rows, int64_t cols, const rr_plan *plan);

/* Static, NUL-terminated name of a status code. */
const char *rr_status_string(int status);

/* ---- Measurement helpers (not part of the method) ------------------------
 * Used by the benchmark to put the operators next to a plain streaming copy
 * of known size (HBM ceiling, counter calibration) and an empty kernel
 * (launch floor). Same ownership and error conventions as above. */

/* dst[i] = src[i] for 0 <= i < n (n floats; no overlap). */
int rr_copy_f32(const float *src, float *dst, int64_t n, void *stream);

/* A streaming kernel of chosen geometry over n floats, for the fastest
 * stream of a given size: copy != 0 copies src to dst; copy == 0 only reads
 * src (dst, at least ceil(n / (4 * packs_per_thread * block)) * block
 * floats, is passed but never written). Each thread moves packs_per_thread
 * (1, 2, 4 or 8) non-temporal 16-byte packs in groups of `block` (256, 512
 * or 1024) threads; other geometries return RR_ERR_UNSUPPORTED. */
int rr_stream_f32(const float *src, float *dst, int64_t n, int32_t copy, int32_t packs_per_thread,
                  int32_t block, void *stream);

/* Launches one workgroup of one wavefront that does nothing. */
int rr_empty_kernel(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWRED_H */

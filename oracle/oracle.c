/*
 * Oracle for the FP32 row-reduction family — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct CPU definitions of what the GPU library
 * computes. Only the test-suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this file's library; the product path never does.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Conventions (identical for every operator):
 *   - x, weights and outputs are row-major, contiguous float32;
 *   - every input is widened exactly to double, every sum, product, square
 *     root, exponential and logarithm is taken in double, and each output is
 *     rounded to float32 exactly once, on the store. This follows the meTile
 *     "Thread Ownership and Software Staging" page, section "Register-tiled
 *     reductions" (FP32 reduction and epilogue, rounding only at the output
 *     store), with double standing in for "at least FP32" so that the oracle
 *     is the exact result up to one final rounding;
 *   - sums run over columns in index order (c = 0, 1, ..., cols-1).
 *
 * The operator list (sum, softmax, RMSNorm, LayerNorm, residual LayerNorm,
 * cross-entropy) is the one the LuisaCompute "Consecutive-worker reduction
 * layout checkpoint" page validates in its section "Evidence and what
 * remains". The pages print RMSNorm's definition only through its name; the
 * other five are the textbook definitions (readings listed per function).
 *
 * The W x V ownership map at the bottom follows the same page, section
 * "Implementation and semantics" (forward map, inverse, and private-slot
 * bound).
 */
#include <math.h>
#include <stdint.h>

/* RMSNorm: y[r,c] = x[r,c] * w[c] / sqrt(mean_c(x[r,c]^2) + eps).
 * Reading: the mean divides by cols; eps is the float32 value passed in,
 * widened (not its decimal spelling). */
int oracle_rmsnorm_f32(const float *x, const float *w, float *y,
                       int64_t rows, int64_t cols, float eps) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        float *yr = y + r * cols;
        double sum_sq = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            double v = (double)xr[c];
            sum_sq += v * v;
        }
        double mean_sq = sum_sq / (double)cols;
        double denom = sqrt(mean_sq + (double)eps);
        for (int64_t c = 0; c < cols; ++c) {
            yr[c] = (float)((double)xr[c] * (double)w[c] / denom);
        }
    }
    return 0;
}

/* Row sum: out[r] = sum_c x[r,c]. */
int oracle_row_sum_f32(const float *x, float *out, int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        double s = 0.0;
        for (int64_t c = 0; c < cols; ++c) s += (double)xr[c];
        out[r] = (float)s;
    }
    return 0;
}

/* Softmax along each row, with the row maximum subtracted first:
 * y[r,c] = exp(x[r,c] - m_r) / sum_k exp(x[r,k] - m_r), m_r = max_k x[r,k]. */
int oracle_softmax_f32(const float *x, float *y, int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        float *yr = y + r * cols;
        double m = (double)xr[0];
        for (int64_t c = 1; c < cols; ++c)
            if ((double)xr[c] > m) m = (double)xr[c];
        double z = 0.0;
        for (int64_t c = 0; c < cols; ++c) z += exp((double)xr[c] - m);
        for (int64_t c = 0; c < cols; ++c)
            yr[c] = (float)(exp((double)xr[c] - m) / z);
    }
    return 0;
}

/* LayerNorm over one row held as doubles; shared by the two LayerNorm
 * entry points below. Reading: population (biased) variance, divisor cols;
 * eps inside the square root; mean and variance each from its own pass. */
static void layernorm_row(const double *h, const float *gamma, const float *beta,
                          float *yr, int64_t cols, float eps) {
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += h[c];
    double mean = s / (double)cols;
    double ss = 0.0;
    for (int64_t c = 0; c < cols; ++c) ss += (h[c] - mean) * (h[c] - mean);
    double var = ss / (double)cols;
    double denom = sqrt(var + (double)eps);
    for (int64_t c = 0; c < cols; ++c)
        yr[c] = (float)((h[c] - mean) / denom * (double)gamma[c] + (double)beta[c]);
}

/* LayerNorm: y = (x - mean) / sqrt(var + eps) * gamma + beta, per row.
 * `scratch` holds cols doubles (caller-owned). */
int oracle_layernorm_f32(const float *x, const float *gamma, const float *beta, float *y,
                         int64_t rows, int64_t cols, float eps, double *scratch) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        for (int64_t c = 0; c < cols; ++c) scratch[c] = (double)xr[c];
        layernorm_row(scratch, gamma, beta, y + r * cols, cols, eps);
    }
    return 0;
}

/* Residual LayerNorm: h = x + residual, rounded to float32 (one float32
 * addition, which is exactly what rounding the double sum gives), then
 * LayerNorm of h. Reading: "added first" means the sum is materialised at
 * the tensors' own precision before normalising. If h_out is not NULL it
 * receives h. `scratch` holds cols doubles. */
int oracle_residual_layernorm_f32(const float *x, const float *residual,
                                  const float *gamma, const float *beta,
                                  float *y, float *h_out, int64_t rows, int64_t cols,
                                  float eps, double *scratch) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        const float *rr = residual + r * cols;
        for (int64_t c = 0; c < cols; ++c) {
            float h = (float)((double)xr[c] + (double)rr[c]);
            scratch[c] = (double)h;
            if (h_out) h_out[r * cols + c] = h;
        }
        layernorm_row(scratch, gamma, beta, y + r * cols, cols, eps);
    }
    return 0;
}

/* Cross-entropy per row with integer class targets:
 * loss[r] = log(sum_c exp(x[r,c] - m_r)) + m_r - x[r, t[r]].
 * Reading: one loss per row, no reduction over rows, no ignored index, no
 * label smoothing or class weights. A target outside [0, cols) gives NaN. */
int oracle_cross_entropy_f32(const float *logits, const int32_t *targets, float *loss,
                             int64_t rows, int64_t cols) {
    if (rows < 0 || cols <= 0) return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = logits + r * cols;
        int32_t t = targets[r];
        if (t < 0 || (int64_t)t >= cols) {
            loss[r] = (float)NAN;
            continue;
        }
        double m = (double)xr[0];
        for (int64_t c = 1; c < cols; ++c)
            if ((double)xr[c] > m) m = (double)xr[c];
        double z = 0.0;
        for (int64_t c = 0; c < cols; ++c) z += exp((double)xr[c] - m);
        loss[r] = (float)(log(z) + m - (double)xr[t]);
    }
    return 0;
}

/* ---- W x V ownership map (consecutive-worker layout) ----------------------
 * W workers cooperate on one row of N elements; each owns runs of V
 * consecutive elements. Element i belongs to worker (i / V) % W, sits in
 * that worker's private slot (i / (W*V)) * V + i % V, and the worker's
 * k-th slot holds element ((k / V) * W + worker) * V + k % V. */

void oracle_owner(int64_t i, int64_t W, int64_t V, int64_t *worker, int64_t *slot) {
    int64_t element = i % V;
    int64_t chunk = i / (W * V);
    *worker = (i / V) % W;
    *slot = chunk * V + element;
}

int64_t oracle_logical_index(int64_t worker, int64_t slot, int64_t W, int64_t V) {
    int64_t chunk = slot / V;
    int64_t element = slot % V;
    return (chunk * W + worker) * V + element;
}

/* Largest number of valid private slots any worker holds for a row of N. */
int64_t oracle_slot_bound(int64_t N, int64_t W, int64_t V) {
    int64_t full = N / (W * V);
    int64_t rem = N % (W * V);
    return full * V + (rem < V ? rem : V);
}

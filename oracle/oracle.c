/*
 * Oracle for the FP32 / BF16 row-reduction family — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct CPU definitions of what the GPU library
 * computes. Only the test-suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this file's library; the product path never does.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Conventions (identical for every operator):
 *   - x, weights and outputs are row-major and contiguous, stored as float32
 *     or as bfloat16 bit patterns (uint16);
 *   - every input is widened exactly to double; every sum, product, square
 *     root, exponential and logarithm is taken in double by the row
 *     definitions below, and each output is rounded to its storage type
 *     exactly once, on the store. This follows the meTile "Thread Ownership
 *     and Software Staging" page, section "Register-tiled reductions" (FP32
 *     reduction and epilogue, rounding only at the output store), with double
 *     standing in for "at least FP32" so that the oracle is the exact result
 *     up to one final rounding;
 *   - sums run over columns in index order (c = 0, 1, ..., cols-1).
 *
 * The operator list (sum, softmax, RMSNorm, LayerNorm, residual LayerNorm,
 * cross-entropy) is the one the LuisaCompute "Consecutive-worker reduction
 * layout checkpoint" page validates in its section "Evidence and what
 * remains". The pages print RMSNorm's definition only through its name; the
 * other five are the textbook definitions (readings listed per function).
 * The bfloat16 entry points serve the same definitions with 16-bit storage
 * (the meTile page measures 16-bit I/O with FP32 arithmetic, section
 * "Measurements and reproduction").
 *
 * The W x V ownership map at the bottom follows the LuisaCompute page,
 * section "Implementation and semantics" (forward map, inverse, and
 * private-slot bound).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage conversions ------------------------------------------------- */

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (8 significant bits, float32
 * exponent range, ties to even), in one step from the exact value. */
uint16_t oracle_bf16_from_double(double v) {
    if (isnan(v)) return 0x7fc0;
    float f;
    if (v == 0.0 || isinf(v)) {
        f = (float)v;
    } else {
        int e;
        frexp(fabs(v), &e);          /* |v| = m * 2^e with 0.5 <= m < 1 */
        int q = e - 8;               /* quantum of an 8-bit significand */
        if (q < -133) q = -133;      /* subnormal range: fixed quantum 2^-133 */
        double r = nearbyint(ldexp(fabs(v), -q));   /* ties to even */
        double res = ldexp(r, q);
        if (res > 3.3895313892515355e38) res = INFINITY;  /* beyond the largest bfloat16 */
        f = (float)copysign(res, v);
    }
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);  /* f is a bfloat16 value: its low half is zero */
}

/* ---- row definitions (double in, double out) ------------------------------ */

/* RMSNorm: y[c] = x[c] * w[c] / sqrt(mean_c(x[c]^2) + eps).
 * Reading: the mean divides by cols; eps is the float32 value passed in,
 * widened (not its decimal spelling). */
static void rmsnorm_row(const double *x, const double *w, double *y, int64_t cols, double eps) {
    double sum_sq = 0.0;
    for (int64_t c = 0; c < cols; ++c) sum_sq += x[c] * x[c];
    double mean_sq = sum_sq / (double)cols;
    double denom = sqrt(mean_sq + eps);
    for (int64_t c = 0; c < cols; ++c) y[c] = x[c] * w[c] / denom;
}

static double sum_row(const double *x, int64_t cols) {
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += x[c];
    return s;
}

/* Softmax with the row maximum subtracted first:
 * y[c] = exp(x[c] - m) / sum_k exp(x[k] - m), m = max_k x[k]. */
static void softmax_row(const double *x, double *y, int64_t cols) {
    double m = x[0];
    for (int64_t c = 1; c < cols; ++c)
        if (x[c] > m) m = x[c];
    double z = 0.0;
    for (int64_t c = 0; c < cols; ++c) z += exp(x[c] - m);
    for (int64_t c = 0; c < cols; ++c) y[c] = exp(x[c] - m) / z;
}

/* LayerNorm: y = (h - mean) / sqrt(var + eps) * gamma + beta. Reading:
 * population (biased) variance, divisor cols; eps inside the square root;
 * mean and variance each from its own pass. */
static void layernorm_row(const double *h, const double *gamma, const double *beta, double *y,
                          int64_t cols, double eps) {
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += h[c];
    double mean = s / (double)cols;
    double ss = 0.0;
    for (int64_t c = 0; c < cols; ++c) ss += (h[c] - mean) * (h[c] - mean);
    double var = ss / (double)cols;
    double denom = sqrt(var + eps);
    for (int64_t c = 0; c < cols; ++c) y[c] = (h[c] - mean) / denom * gamma[c] + beta[c];
}

/* Cross-entropy with an integer class target:
 * loss = log(sum_c exp(x[c] - m)) + m - x[t]. Reading: one loss per row, no
 * reduction over rows, no ignored index, no label smoothing or class
 * weights. A target outside [0, cols) gives NaN. */
static double cross_entropy_row(const double *x, int64_t cols, int32_t t) {
    if (t < 0 || (int64_t)t >= cols) return NAN;
    double m = x[0];
    for (int64_t c = 1; c < cols; ++c)
        if (x[c] > m) m = x[c];
    double z = 0.0;
    for (int64_t c = 0; c < cols; ++c) z += exp(x[c] - m);
    return log(z) + m - x[t];
}

/* ---- storage front ends ---------------------------------------------------- */

typedef enum { F32 = 0, BF16 = 1 } storage;

static double load_elem(const void *p, storage s, int64_t i) {
    return s == F32 ? (double)((const float *)p)[i] : bf16_to_double(((const uint16_t *)p)[i]);
}

static void load_row(const void *p, storage s, int64_t off, int64_t cols, double *dst) {
    for (int64_t c = 0; c < cols; ++c) dst[c] = load_elem(p, s, off + c);
}

static void store_row(void *p, storage s, int64_t off, int64_t cols, const double *src) {
    for (int64_t c = 0; c < cols; ++c) {
        if (s == F32) ((float *)p)[off + c] = (float)src[c];
        else ((uint16_t *)p)[off + c] = oracle_bf16_from_double(src[c]);
    }
}

/* Scratch: four rows of doubles. */
static double *scratch(int64_t cols) { return (double *)malloc(sizeof(double) * 4 * (size_t)cols); }

static int rmsnorm_any(const void *x, const void *w, void *y, int64_t rows, int64_t cols, float eps,
                       storage s) {
    if (rows < 0 || cols <= 0) return 1;
    double *buf = scratch(cols);
    if (!buf) return 2;
    double *xr = buf, *wr = buf + cols, *yr = buf + 2 * cols;
    load_row(w, s, 0, cols, wr);
    for (int64_t r = 0; r < rows; ++r) {
        load_row(x, s, r * cols, cols, xr);
        rmsnorm_row(xr, wr, yr, cols, (double)eps);
        store_row(y, s, r * cols, cols, yr);
    }
    free(buf);
    return 0;
}

static int row_sum_any(const void *x, float *out, int64_t rows, int64_t cols, storage s) {
    if (rows < 0 || cols <= 0) return 1;
    double *xr = scratch(cols);
    if (!xr) return 2;
    for (int64_t r = 0; r < rows; ++r) {
        load_row(x, s, r * cols, cols, xr);
        out[r] = (float)sum_row(xr, cols);
    }
    free(xr);
    return 0;
}

static int softmax_any(const void *x, void *y, int64_t rows, int64_t cols, storage s) {
    if (rows < 0 || cols <= 0) return 1;
    double *buf = scratch(cols);
    if (!buf) return 2;
    double *xr = buf, *yr = buf + cols;
    for (int64_t r = 0; r < rows; ++r) {
        load_row(x, s, r * cols, cols, xr);
        softmax_row(xr, yr, cols);
        store_row(y, s, r * cols, cols, yr);
    }
    free(buf);
    return 0;
}

/* LayerNorm of x, or of h = x + residual rounded to the storage type when
 * residual is not NULL. Reading: "added first" means the sum is materialised
 * at the tensors' own precision before normalising (one rounding of the exact
 * sum); h_out, if not NULL, receives it. */
static int layernorm_any(const void *x, const void *residual, const void *gamma, const void *beta,
                         void *y, void *h_out, int64_t rows, int64_t cols, float eps, storage s) {
    if (rows < 0 || cols <= 0) return 1;
    double *buf = scratch(cols);
    if (!buf) return 2;
    double *hr = buf, *gr = buf + cols, *br = buf + 2 * cols, *yr = buf + 3 * cols;
    load_row(gamma, s, 0, cols, gr);
    load_row(beta, s, 0, cols, br);
    for (int64_t r = 0; r < rows; ++r) {
        load_row(x, s, r * cols, cols, hr);
        if (residual) {
            for (int64_t c = 0; c < cols; ++c) {
                double sum = hr[c] + load_elem(residual, s, r * cols + c);
                hr[c] = s == F32 ? (double)(float)sum : bf16_to_double(oracle_bf16_from_double(sum));
            }
            if (h_out) store_row(h_out, s, r * cols, cols, hr);
        }
        layernorm_row(hr, gr, br, yr, cols, (double)eps);
        store_row(y, s, r * cols, cols, yr);
    }
    free(buf);
    return 0;
}

static int cross_entropy_any(const void *x, const int32_t *targets, float *loss, int64_t rows,
                             int64_t cols, storage s) {
    if (rows < 0 || cols <= 0) return 1;
    double *xr = scratch(cols);
    if (!xr) return 2;
    for (int64_t r = 0; r < rows; ++r) {
        load_row(x, s, r * cols, cols, xr);
        loss[r] = (float)cross_entropy_row(xr, cols, targets[r]);
    }
    free(xr);
    return 0;
}

/* ---- exported entry points ------------------------------------------------ */

int oracle_rmsnorm_f32(const float *x, const float *w, float *y, int64_t rows, int64_t cols, float eps) {
    return rmsnorm_any(x, w, y, rows, cols, eps, F32);
}
int oracle_row_sum_f32(const float *x, float *out, int64_t rows, int64_t cols) {
    return row_sum_any(x, out, rows, cols, F32);
}
int oracle_softmax_f32(const float *x, float *y, int64_t rows, int64_t cols) {
    return softmax_any(x, y, rows, cols, F32);
}
int oracle_layernorm_f32(const float *x, const float *gamma, const float *beta, float *y,
                         int64_t rows, int64_t cols, float eps) {
    return layernorm_any(x, NULL, gamma, beta, y, NULL, rows, cols, eps, F32);
}
int oracle_residual_layernorm_f32(const float *x, const float *residual, const float *gamma,
                                  const float *beta, float *y, float *h_out, int64_t rows,
                                  int64_t cols, float eps) {
    return layernorm_any(x, residual, gamma, beta, y, h_out, rows, cols, eps, F32);
}
int oracle_cross_entropy_f32(const float *logits, const int32_t *targets, float *loss, int64_t rows,
                             int64_t cols) {
    return cross_entropy_any(logits, targets, loss, rows, cols, F32);
}

int oracle_rmsnorm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y, int64_t rows, int64_t cols,
                        float eps) {
    return rmsnorm_any(x, w, y, rows, cols, eps, BF16);
}
int oracle_row_sum_bf16(const uint16_t *x, float *out, int64_t rows, int64_t cols) {
    return row_sum_any(x, out, rows, cols, BF16);
}
int oracle_softmax_bf16(const uint16_t *x, uint16_t *y, int64_t rows, int64_t cols) {
    return softmax_any(x, y, rows, cols, BF16);
}
int oracle_layernorm_bf16(const uint16_t *x, const uint16_t *gamma, const uint16_t *beta, uint16_t *y,
                          int64_t rows, int64_t cols, float eps) {
    return layernorm_any(x, NULL, gamma, beta, y, NULL, rows, cols, eps, BF16);
}
int oracle_residual_layernorm_bf16(const uint16_t *x, const uint16_t *residual, const uint16_t *gamma,
                                   const uint16_t *beta, uint16_t *y, uint16_t *h_out, int64_t rows,
                                   int64_t cols, float eps) {
    return layernorm_any(x, residual, gamma, beta, y, h_out, rows, cols, eps, BF16);
}
int oracle_cross_entropy_bf16(const uint16_t *logits, const int32_t *targets, float *loss, int64_t rows,
                              int64_t cols) {
    return cross_entropy_any(logits, targets, loss, rows, cols, BF16);
}

/* ---- one very long float32 row, selected outputs ---------------------------
 * The same definitions as rmsnorm_row, sum_row and softmax_row, evaluated
 * for a single row read element by element from its float32 storage (no
 * float64 copy of the row), with outputs only at the n columns idx[] asks
 * for: rows of up to 2^31 columns then need no row-sized scratch. The row
 * statistics accumulate in the same order as the full-row versions. */

int oracle_rmsnorm_f32_sampled(const float *x, const float *w, int64_t cols, float eps,
                               const int64_t *idx, int64_t n, float *y) {
    if (cols <= 0 || n < 0) return 1;
    double sum_sq = 0.0;
    for (int64_t c = 0; c < cols; ++c) sum_sq += (double)x[c] * (double)x[c];
    double denom = sqrt(sum_sq / (double)cols + (double)eps);
    for (int64_t k = 0; k < n; ++k) {
        if (idx[k] < 0 || idx[k] >= cols) return 1;
        y[k] = (float)((double)x[idx[k]] * (double)w[idx[k]] / denom);
    }
    return 0;
}

int oracle_row_sum_f32_long(const float *x, int64_t cols, float *out) {
    if (cols <= 0) return 1;
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += (double)x[c];
    *out = (float)s;
    return 0;
}

int oracle_softmax_f32_sampled(const float *x, int64_t cols, const int64_t *idx, int64_t n, float *y) {
    if (cols <= 0 || n < 0) return 1;
    double m = (double)x[0];
    for (int64_t c = 1; c < cols; ++c)
        if ((double)x[c] > m) m = (double)x[c];
    double z = 0.0;
    for (int64_t c = 0; c < cols; ++c) z += exp((double)x[c] - m);
    for (int64_t k = 0; k < n; ++k) {
        if (idx[k] < 0 || idx[k] >= cols) return 1;
        y[k] = (float)(exp((double)x[idx[k]] - m) / z);
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

/*
 * CPU oracle for the normalization forward passes — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's cpu_baseline leg
 * may call this code.  The GPU library shares nothing with it: no headers,
 * no helpers, no constants.  Every function is the plain definition of the
 * operation written out in double precision:
 *   - inputs arrive as double (the callers promote fp32 data exactly),
 *   - eps and negative_slope are the fp32 values the GPU library receives,
 *     promoted to double by the caller,
 *   - every sum is a sequential left-to-right loop (no blocking, no
 *     reordering), statistics are two-pass (mean first, then the sum of
 *     squared deviations),
 *   - results are returned unrounded (double); rounding to fp32, if wanted,
 *     is the caller's.
 * Parallelism is only across independent segments (samples, rows,
 * positions), never inside a sum, so results do not depend on the thread
 * count.
 *
 * Sources ("pages" are three POPCORNBENCH agent transcripts; a "turn" is one
 * agent message on a page):
 *   LN page  = "Kimi-K2.6 l1_p40" (LayerNorm over (64,256,256) per sample)
 *   GN page  = "Kimi-K2.6 l2_p62" (fc -> GroupNorm -> LeakyReLU -> x + x)
 *   RMS page = "Kimi-K2.6 l1_p36" (RMSNorm along dim 1 of NCHW)
 *
 * Every function here is pinned by tests that do not go through this file:
 * exact-rational brute force on tiny inputs, closed forms, invariants and
 * special cases (see tests/test_oracle_*.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * LayerNorm (LN page, turn 1, the problem analysis: statistics over all
 * trailing dims of one sample, population variance with no Bessel
 * correction, eps added to the variance inside the square root, elementwise
 * weight and bias of normalized_shape; turn 2 allows either affine tensor to
 * be absent, meaning weight 1 / bias 0).
 *
 * x, y: [outer, inner] row-major.  w, b: [inner] or NULL.
 * mean_out, var_out: [outer] or NULL.
 */
void oracle_ln(const double* x, const double* w, const double* b,
               int64_t outer, int64_t inner, double eps,
               double* y, double* mean_out, double* var_out)
{
    if (outer <= 0 || inner <= 0) return;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < outer; ++r) {
        const double* xr = x + r * inner;
        double* yr = y ? y + r * inner : NULL;
        double sum = 0.0;
        for (int64_t i = 0; i < inner; ++i) sum += xr[i];
        const double mean = sum / (double)inner;
        double ssd = 0.0;
        for (int64_t i = 0; i < inner; ++i) {
            const double d = xr[i] - mean;
            ssd += d * d;
        }
        const double var = ssd / (double)inner;
        const double denom = sqrt(var + eps);
        if (mean_out) mean_out[r] = mean;
        if (var_out) var_out[r] = var;
        if (!yr) continue;
        for (int64_t i = 0; i < inner; ++i) {
            double v = (xr[i] - mean) / denom;
            if (w) v = v * w[i];
            if (b) v = v + b[i];
            yr[i] = v;
        }
    }
}

/*
 * GroupNorm -> LeakyReLU -> x + x (GN page, turn 1: the fc output [N, C] is
 * split into num_groups groups of M = C / num_groups *contiguous* channels;
 * each (row, group) gets its own mean and population variance; per-channel
 * gamma/beta; then LeakyReLU with negative_slope; then the tensor is added
 * to itself).  gamma/beta may be NULL (identity affine).
 *
 * x, y: [N, C] row-major; gamma, beta: [C] or NULL; C % G == 0 is the
 * caller's precondition.  mean_out, var_out: [N, G] or NULL.
 */
void oracle_gn_lrelu_x2(const double* x, const double* gamma, const double* beta,
                        int64_t N, int64_t C, int64_t G, double eps, double slope,
                        double* y, double* mean_out, double* var_out)
{
    if (N <= 0 || C <= 0 || G <= 0 || C % G != 0) return;
    const int64_t M = C / G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const double* xg = x + n * C + g * M;
            double sum = 0.0;
            for (int64_t j = 0; j < M; ++j) sum += xg[j];
            const double mean = sum / (double)M;
            double ssd = 0.0;
            for (int64_t j = 0; j < M; ++j) {
                const double d = xg[j] - mean;
                ssd += d * d;
            }
            const double var = ssd / (double)M;
            const double denom = sqrt(var + eps);
            if (mean_out) mean_out[n * G + g] = mean;
            if (var_out) var_out[n * G + g] = var;
            if (!y) continue;
            for (int64_t j = 0; j < M; ++j) {
                const int64_t c = g * M + j;
                double z = (xg[j] - mean) / denom;
                if (gamma) z = z * gamma[c];
                if (beta) z = z + beta[c];
                const double a = z > 0.0 ? z : slope * z;
                y[n * C + c] = a + a;
            }
        }
    }
}

/*
 * RMSNorm along dim 1 (RMS page, turn 1 and the reference model quoted in
 * turn 2: rms = sqrt(mean over the feature dim of x^2, plus eps), output =
 * x / rms; no affine).  The tensor is viewed as [B, C, S] with S the product
 * of the trailing dims, so the C values of one position (b, s) sit S
 * elements apart.
 *
 * x, y: [B, C, S] row-major.  ms_out: [B, S] mean of squares, or NULL.
 */
void oracle_rms_ch(const double* x, int64_t B, int64_t C, int64_t S, double eps,
                   double* y, double* ms_out)
{
    if (B <= 0 || C <= 0 || S <= 0) return;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < B * S; ++p) {
        const int64_t b = p / S, s = p % S;
        const double* xp = x + b * C * S + s;
        double sumsq = 0.0;
        for (int64_t c = 0; c < C; ++c) sumsq += xp[c * S] * xp[c * S];
        const double ms = sumsq / (double)C;
        const double rms = sqrt(ms + eps);
        if (ms_out) ms_out[p] = ms;
        if (!y) continue;
        double* yp = y + b * C * S + s;
        for (int64_t c = 0; c < C; ++c) yp[c * S] = xp[c * S] / rms;
    }
}

/*
 * Linear layer (GN page, turn 1: y = x W^T + b with x [N, K], W [Cout, K]
 * and b [Cout]).  Each output is one sequential dot product over k.
 * bias may be NULL.
 */
void oracle_fc(const double* x, const double* W, const double* bias,
               int64_t N, int64_t K, int64_t Cout, double* h)
{
    if (N <= 0 || K < 0 || Cout <= 0) return;  /* K == 0: the empty sum, h = bias */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t c = 0; c < Cout; ++c) {
            const double* xr = x + n * K;
            const double* wr = W + c * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xr[k] * wr[k];
            if (bias) acc += bias[c];
            h[n * Cout + c] = acc;
        }
    }
}

/* Number of threads an OpenMP parallel region here uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

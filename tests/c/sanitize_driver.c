/*
 * Host code under AddressSanitizer and UndefinedBehaviorSanitizer, no GPU:
 *   - every validation path of the C ABI (calls that must return an error
 *     before anything is launched) and the empty-work no-ops, against a
 *     libnormfwd whose host code is built with the sanitizers;
 *   - the CPU oracle (built with the sanitizers) on small problems of every
 *     operation, with invariants checked.
 * Exit status 0 = no sanitizer report and every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "normfwd.h"

void oracle_ln(const double* x, const double* w, const double* b, int64_t outer, int64_t inner, double eps,
               double* y, double* mean_out, double* var_out);
void oracle_gn_lrelu_x2(const double* x, const double* gamma, const double* beta, int64_t N, int64_t C, int64_t G,
                        double eps, double slope, double* y, double* mean_out, double* var_out);
void oracle_rms_ch(const double* x, int64_t B, int64_t C, int64_t S, double eps, double* y, double* ms_out);
void oracle_fc(const double* x, const double* W, const double* bias, int64_t N, int64_t K, int64_t Cout, double* h);

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, normfwd_last_error()); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

static double* rnd(size_t n, unsigned seed)
{
    double* p = (double*)malloc(n * sizeof(double));
    uint64_t s = 0x9E3779B97F4A7C15ull ^ seed;
    for (size_t i = 0; i < n; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        p[i] = (double)((s >> 40) * (1.0 / 16777216.0)) * 4.0 - 2.0;
    }
    return p;
}

int main(void)
{
    /* ---- C ABI: rejected before any launch */
    float* fake = (float*)(uintptr_t)0x100000;
    void* ws = (void*)(uintptr_t)0x200000;
    EXPECT(ln_forward(NULL, NULL, NULL, fake, 2, 8, 1e-5f, ws, 1 << 20, NULL, NULL, 0, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(ln_forward(fake, NULL, NULL, fake, 2, 8, 1e-5f, NULL, 1 << 20, NULL, NULL, 0, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(ln_forward(fake, NULL, NULL, fake, 2, 8, 1e-5f, ws, 1 << 20, NULL, NULL, 9, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(ln_forward(fake, NULL, NULL, fake, (1 << 22) + 1, 8, 1e-5f, ws, 1 << 20, NULL, NULL, 0, NULL) ==
           NORMFWD_ERR_UNSUPPORTED);
    EXPECT(ln_forward(fake, NULL, NULL, fake, 16, 4194304, 1e-5f, ws, 100, NULL, NULL, 0, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(ln_forward_noalloc(fake, NULL, NULL, fake, 1024, 1 << 20, 1e-5f, NULL, NULL, 3, NULL) ==
           NORMFWD_ERR_UNSUPPORTED);
    EXPECT(ln_forward_stats(fake, 16, 4194304, 1e-5f, ws, 100, NULL, NULL, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(ln_forward_apply(fake, NULL, NULL, NULL, 16, 4194304, ws, 1 << 30, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(ln_forward_workspace_init(NULL, 1024, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(ln_forward_workspace_check((void*)(uintptr_t)0x200010, 1024, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(ln_forward_workspace_size(16, 4194304) > 0 && ln_forward_workspace_size(0, 5) == 0);
    EXPECT(gn_lrelu_x2_forward(fake, NULL, NULL, fake, 4, 10, 3, 1e-5f, 0.01f, NULL, NULL, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(gn_lrelu_x2_forward(fake, NULL, NULL, fake, 4, 12, 3, 1e-5f, 0.01f, fake, NULL, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(gn_lrelu_x2_forward(fake, NULL, NULL, fake, 4, (1 << 30) + 4, 4, 1e-5f, 0.01f, NULL, NULL, NULL) ==
           NORMFWD_ERR_UNSUPPORTED);
    EXPECT(rmsnorm_ch_forward(fake, fake, 2, 0, 4, 1e-5f, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(rmsnorm_ch_forward(fake, fake, 1, 3, (1 << 26) + 4, 1e-5f, NULL) == NORMFWD_ERR_UNSUPPORTED);
    EXPECT(rmsnorm_ch_forward_strided(fake, fake, 2, 3, 4, 12, 4, 12, 3, 1e-5f, NULL, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(rmsnorm_ch_forward_strided(fake, fake, 2, 3, 4, -1, 4, 12, 4, 1e-5f, NULL, NULL) == NORMFWD_ERR_UNSUPPORTED);
    EXPECT(rmsnorm_ch_forward_strided(fake, fake, 3, 3, 4, INT64_MAX / 2, 4, 12, 4, 1e-5f, NULL, NULL) ==
           NORMFWD_ERR_UNSUPPORTED);
    EXPECT(fc_gn_forward(fake, fake, NULL, NULL, NULL, fake, 1024, 8192, 8192, 500, 1e-5f, 0.01f, ws, 1u << 30,
                         NULL, NULL, NULL) == NORMFWD_ERR_INVALID);
    EXPECT(fc_gn_forward(fake, fake, NULL, NULL, NULL, fake, 1024, 8192, 8192, 512, 1e-5f, 0.01f, ws, 4, NULL,
                         NULL, NULL) == NORMFWD_ERR_WORKSPACE);
    EXPECT(normfwd_copy_reference(fake, fake, 1, 1, 6, 0, NULL) == NORMFWD_ERR_UNSUPPORTED);
    EXPECT(normfwd_copy_reference(fake, fake, 1, 1, 8, 5, NULL) == NORMFWD_ERR_INVALID);
    /* empty work: OK without touching any pointer */
    EXPECT(ln_forward(NULL, NULL, NULL, NULL, 0, 8, 1e-5f, NULL, 0, NULL, NULL, 1, NULL) == NORMFWD_OK);
    EXPECT(ln_forward_noalloc(NULL, NULL, NULL, NULL, 0, 8, 1e-5f, NULL, NULL, 3, NULL) == NORMFWD_OK);
    EXPECT(gn_lrelu_x2_forward(NULL, NULL, NULL, NULL, 0, 64, 4, 1e-5f, 0.01f, NULL, NULL, NULL) == NORMFWD_OK);
    EXPECT(rmsnorm_ch_forward_strided(NULL, NULL, 0, 3, 4, 12, 4, 12, 4, 1e-5f, NULL, NULL) == NORMFWD_OK);
    EXPECT(fc_gn_forward(NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 128, 8, 1e-5f, 0.01f, NULL, 0, NULL, NULL,
                         NULL) == NORMFWD_OK);
    for (int s = -1; s < 7; ++s) EXPECT(normfwd_status_string(s) != NULL);

    /* ---- oracle on small problems */
    {
        const int64_t outer = 3, inner = 37;
        double *x = rnd((size_t)(outer * inner), 1), *w = rnd((size_t)inner, 2), *b = rnd((size_t)inner, 3);
        double* y = (double*)malloc(sizeof(double) * (size_t)(outer * inner));
        double mean[3], var[3];
        oracle_ln(x, NULL, NULL, outer, inner, 1e-5, y, mean, var);
        for (int64_t r = 0; r < outer; ++r) {
            double s = 0.0;
            for (int64_t i = 0; i < inner; ++i) s += y[r * inner + i];
            EXPECT(fabs(s) < 1e-10 && var[r] > 0.0);
        }
        oracle_ln(x, w, b, outer, inner, 1e-5, y, NULL, NULL);
        free(x), free(w), free(b), free(y);
    }
    {
        const int64_t N = 4, C = 24, G = 6;
        double *x = rnd((size_t)(N * C), 4), *g = rnd((size_t)C, 5), *bt = rnd((size_t)C, 6);
        double* y = (double*)malloc(sizeof(double) * (size_t)(N * C));
        double mean[24], var[24];
        oracle_gn_lrelu_x2(x, g, bt, N, C, G, 1e-5, 0.01, y, mean, var);
        for (int i = 0; i < N * G; ++i) EXPECT(var[i] >= 0.0);
        free(x), free(g), free(bt), free(y);
    }
    {
        const int64_t B = 2, C = 5, S = 7;
        double* x = rnd((size_t)(B * C * S), 7);
        double* y = (double*)malloc(sizeof(double) * (size_t)(B * C * S));
        double ms[14];
        oracle_rms_ch(x, B, C, S, 1e-5, y, ms);
        for (int i = 0; i < B * S; ++i) EXPECT(ms[i] > 0.0);
        free(x), free(y);
    }
    {
        const int64_t N = 3, K = 9, Co = 4;
        double *x = rnd((size_t)(N * K), 8), *W = rnd((size_t)(Co * K), 9), *bb = rnd((size_t)Co, 10);
        double* h = (double*)malloc(sizeof(double) * (size_t)(N * Co));
        oracle_fc(x, W, bb, N, K, Co, h);
        double want = bb[0];
        for (int64_t k = 0; k < K; ++k) want += x[k] * W[k];
        EXPECT(fabs(h[0] - want) < 1e-12);
        oracle_fc(x, W, NULL, N, 0, Co, h); /* K = 0: h = 0 without a bias */
        EXPECT(h[0] == 0.0);
        free(x), free(W), free(bb), free(h);
    }
    if (fails) {
        printf("sanitize_driver: %d failures\n", fails);
        return 1;
    }
    printf("sanitize_driver: ok\n");
    return 0;
}

/* Drives the CPU oracle (oracle/gdr_oracle.c) through every gate and decay
 * mode, head and column selections, one and several threads, and its
 * argument checks, in a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use after free,
 * leak or undefined operation aborts the run. It also checks two facts the
 * pages fix, so that the run exercises real arithmetic: with beta = 0 and no
 * decay the state passes through unchanged, and a selection of heads and
 * columns gives exactly the full run's values there. Exit status 0 when
 * every check holds. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdr_oracle_recurrent(int B, int T, int Hqk, int Hv, int dk, int dv, const double *q, const double *k,
                         const double *v, const double *g, int decay, const double *beta, const double *bg,
                         const double *wg, double scale, const double *S0, double *o, double *ST, const int *heads,
                         int n_heads, int col0, int col1, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    return p;
}

static int failures = 0;
#define CHECK(cond, what)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "check failed: %s\n", what);   \
            ++failures;                                    \
        }                                                  \
    } while (0)

int main(void) {
    const int B = 2, T = 37, Hqk = 2, Hv = 4, d = 8;
    const size_t nqk = (size_t)B * T * Hqk * d, nv = (size_t)B * T * Hv * d, ns = (size_t)B * Hv * d * d;
    double *q = arr(nqk, -1, 1), *k = arr(nqk, -0.3, 0.3), *v = arr(nv, -1, 1);
    double *gs = arr((size_t)B * T * Hv, -0.5, 0.0), *gc = arr(nv, -3.0, 0.0), *beta = arr((size_t)B * T * Hv, 0, 1);
    double *bg = arr(nv, 0, 1), *wg = arr(nv, 0, 1), *S0 = arr(ns, -0.1, 0.1);
    double *o = (double *)calloc(nv, sizeof(double)), *ST = (double *)calloc(ns, sizeof(double));
    double *o2 = (double *)calloc(nv, sizeof(double)), *ST2 = (double *)calloc(ns, sizeof(double));
    const double *gsel[3] = {NULL, gs, gc};
    for (int decay = 0; decay < 3; ++decay)
        for (int tied = 0; tied < 2; ++tied)
            for (int threads = 1; threads <= 3; threads += 2) {
                int rc = gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, gsel[decay], decay, tied ? beta : NULL,
                                              tied ? NULL : bg, tied ? NULL : wg, 0.5, S0, o, ST, NULL, 0, 0, d,
                                              threads);
                CHECK(rc == 0, "full run");
                for (size_t i = 0; i < nv; ++i) CHECK(isfinite(o[i]), "finite output");
                /* A selection of heads and columns gives the full run's values there. */
                const int heads[2] = {3, 1};
                memset(o2, 0, sizeof(double) * nv);
                rc = gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, gsel[decay], decay, tied ? beta : NULL,
                                          tied ? NULL : bg, tied ? NULL : wg, 0.5, S0, o2, ST2, heads, 2, 2, 7,
                                          threads);
                CHECK(rc == 0, "selected run");
                for (int b = 0; b < B; ++b)
                    for (int t = 0; t < T; ++t)
                        for (int hi = 0; hi < 2; ++hi)
                            for (int c = 2; c < 7; ++c) {
                                const size_t i = (((size_t)b * T + t) * Hv + heads[hi]) * d + c;
                                CHECK(o2[i] == o[i], "selection equals the full run");
                            }
            }
    /* beta = 0, no decay: the state passes through unchanged. */
    double *zero = (double *)calloc((size_t)B * T * Hv, sizeof(double));
    int rc = gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, NULL, 0, zero, NULL, NULL, 1.0, S0, o, ST, NULL, 0, 0,
                                  d, 2);
    CHECK(rc == 0, "beta = 0 run");
    for (size_t i = 0; i < ns; ++i) CHECK(ST[i] == S0[i], "beta = 0 keeps the state");
    /* T = 0 and argument checks. */
    CHECK(gdr_oracle_recurrent(B, 0, Hqk, Hv, d, d, q, k, v, NULL, 0, beta, NULL, NULL, 1.0, S0, o, ST, NULL, 0, 0, d,
                               1) == 0, "T = 0");
    CHECK(gdr_oracle_recurrent(B, T, 3, Hv, d, d, q, k, v, NULL, 0, beta, NULL, NULL, 1.0, S0, o, ST, NULL, 0, 0, d,
                               1) == -1, "H_v not a multiple of H_qk");
    CHECK(gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, NULL, 1, beta, NULL, NULL, 1.0, S0, o, ST, NULL, 0, 0, d,
                               1) == -1, "scalar decay without g");
    CHECK(gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, NULL, 0, beta, bg, NULL, 1.0, S0, o, ST, NULL, 0, 0, d,
                               1) == -1, "beta with b");
    const int bad[1] = {Hv};
    CHECK(gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, NULL, 0, beta, NULL, NULL, 1.0, S0, o, ST, bad, 1, 0, d,
                               1) == -1, "head out of range");
    CHECK(gdr_oracle_recurrent(B, T, Hqk, Hv, d, d, q, k, v, NULL, 0, beta, NULL, NULL, 1.0, S0, o, ST, NULL, 0, 3, 3,
                               1) == -1, "empty column range");
    free(q); free(k); free(v); free(gs); free(gc); free(beta); free(bg); free(wg); free(S0);
    free(o); free(ST); free(o2); free(ST2); free(zero);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}

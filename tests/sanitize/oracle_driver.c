/*
 * oracle_driver.c -- runs the fp64 C oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure).  Covers packed sequences
 * with empty ones, a NULL initial state, column blocks that do not divide d_v,
 * the decode step, and the argument checks; verifies two closed forms so that
 * a silent out-of-bounds read would also show up as a wrong number.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_prefill(int32_t n_seqs, const int64_t *cu_seqlens, int32_t H, int32_t dk,
                       int32_t dv, const double *q, const double *k, const double *v,
                       const double *g, const double *beta, double scale, const double *s0,
                       double *o, double *s_final, int32_t col_block, int32_t n_threads);
int kda_oracle_decode_step(int32_t n_sessions, int32_t H, int32_t dk, int32_t dv,
                           const double *q, const double *k, const double *v, const double *g,
                           const double *beta, double scale, double *state, double *o,
                           int32_t n_threads);

static int checks = 0;
#define CHECK(c)                                                                   \
    do {                                                                           \
        ++checks;                                                                  \
        if (!(c)) {                                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);   \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

static double *alloc(size_t n, unsigned *seed) {
    double *p = (double *)malloc(n * sizeof(double));
    size_t i;
    for (i = 0; i < n; ++i) p[i] = (double)rand_r(seed) / RAND_MAX - 0.5;
    return p;
}

int main(void) {
    enum { H = 3, DK = 8, DV = 7, N = 4 };
    const int64_t cu[N + 1] = {0, 5, 5, 17, 18};   /* lengths 5, 0, 12, 1 */
    const int T = 18;
    unsigned seed = 12345;
    double *q = alloc((size_t)T * H * DK, &seed), *k = alloc((size_t)T * H * DK, &seed);
    double *v = alloc((size_t)T * H * DV, &seed), *g = alloc((size_t)T * H * DK, &seed);
    double *beta = alloc((size_t)T * H, &seed), *s0 = alloc((size_t)N * H * DK * DV, &seed);
    double *o = calloc((size_t)T * H * DV, sizeof(double));
    double *o2 = calloc((size_t)T * H * DV, sizeof(double));
    double *sf = calloc((size_t)N * H * DK * DV, sizeof(double));
    double *sf2 = calloc((size_t)N * H * DK * DV, sizeof(double));
    size_t i;
    int t, h, r, c;
    for (i = 0; i < (size_t)T * H * DK; ++i) g[i] = -fabs(g[i]);   /* log-decays <= 0 */

    /* Column blocks of 3 (not dividing 7) and one block give the same numbers. */
    CHECK(kda_oracle_prefill(N, cu, H, DK, DV, q, k, v, g, beta, 0.35, s0, o, sf, 3, 2) == 0);
    CHECK(kda_oracle_prefill(N, cu, H, DK, DV, q, k, v, g, beta, 0.35, s0, o2, sf2, 0, 1) == 0);
    for (i = 0; i < (size_t)T * H * DV; ++i) CHECK(o[i] == o2[i]);
    for (i = 0; i < (size_t)N * H * DK * DV; ++i) CHECK(sf[i] == sf2[i]);
    /* The empty sequence returns its initial state exactly. */
    for (i = 0; i < (size_t)H * DK * DV; ++i) CHECK(sf[(size_t)1 * H * DK * DV + i] == s0[(size_t)1 * H * DK * DV + i]);
    /* NULL initial state. */
    CHECK(kda_oracle_prefill(N, cu, H, DK, DV, q, k, v, g, beta, 0.35, NULL, o2, sf2, 4, 0) == 0);

    /* beta = 0: pure per-row decay of S0, closed form. */
    {
        double *b0 = calloc((size_t)T * H, sizeof(double));
        CHECK(kda_oracle_prefill(N, cu, H, DK, DV, q, k, v, g, b0, 0.35, s0, o2, sf2, 2, 0) == 0);
        for (h = 0; h < H; ++h)
            for (r = 0; r < DK; ++r) {
                double sum = 0.0;
                for (t = (int)cu[2]; t < (int)cu[3]; ++t) sum += g[((size_t)t * H + h) * DK + r];
                for (c = 0; c < DV; ++c) {
                    size_t at = (((size_t)2 * H + h) * DK + r) * DV + c;
                    CHECK(fabs(sf2[at] - exp(sum) * s0[at]) <= 1e-12 * (1.0 + fabs(s0[at])));
                }
            }
        free(b0);
    }

    /* Decode: one step equals a one-token prefill. */
    {
        int64_t cu1[2] = {0, 1};
        double *st = malloc((size_t)H * DK * DV * sizeof(double));
        double *od = calloc((size_t)H * DV, sizeof(double));
        for (i = 0; i < (size_t)H * DK * DV; ++i) st[i] = s0[i];
        CHECK(kda_oracle_decode_step(1, H, DK, DV, q, k, v, g, beta, 0.35, st, od, 3) == 0);
        CHECK(kda_oracle_prefill(1, cu1, H, DK, DV, q, k, v, g, beta, 0.35, s0, o2, sf2, 0, 0) == 0);
        for (i = 0; i < (size_t)H * DV; ++i) CHECK(od[i] == o2[i]);
        for (i = 0; i < (size_t)H * DK * DV; ++i) CHECK(st[i] == sf2[i]);
        free(st);
        free(od);
    }

    /* Argument checks: rejected, nothing written. */
    {
        const int64_t bad_start[2] = {1, 5}, decreasing[3] = {0, 5, 4};
        CHECK(kda_oracle_prefill(1, bad_start, H, DK, DV, q, k, v, g, beta, 1.0, NULL, o2, sf2, 0, 0) == -1);
        CHECK(kda_oracle_prefill(2, decreasing, H, DK, DV, q, k, v, g, beta, 1.0, NULL, o2, sf2, 0, 0) == -1);
        CHECK(kda_oracle_prefill(N, cu, 0, DK, DV, q, k, v, g, beta, 1.0, NULL, o2, sf2, 0, 0) == -1);
        CHECK(kda_oracle_prefill(N, cu, H, DK, DV, NULL, k, v, g, beta, 1.0, NULL, o2, sf2, 0, 0) == -1);
        CHECK(kda_oracle_prefill(N, NULL, H, DK, DV, q, k, v, g, beta, 1.0, NULL, o2, sf2, 0, 0) == -1);
        CHECK(kda_oracle_decode_step(1, H, DK, DV, q, NULL, v, g, beta, 1.0, sf2, o2, 0) == -1);
        CHECK(kda_oracle_decode_step(-1, H, DK, DV, q, k, v, g, beta, 1.0, sf2, o2, 0) == -1);
    }
    free(q); free(k); free(v); free(g); free(beta); free(s0);
    free(o); free(o2); free(sf); free(sf2);
    printf("oracle driver: %d checks passed\n", checks);
    return 0;
}

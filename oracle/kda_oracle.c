/*
 * kda_oracle.c -- fp64 token-by-token Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct CPU
 * definition that the GPU path is checked against.  Only tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library, and includes nothing from it.
 *
 * What it computes (one head, column vectors, key-by-value state S, d_k x d_v):
 *
 *   retain   S_bar = Diag(a_t) S_{t-1},       a_t = exp(g_t), g_t = log a_t <= 0
 *   predict  v_hat = S_bar^T k_t
 *   correct  S_t   = S_bar + beta_t k_t (v_t - v_hat)^T
 *   read     o_t   = S_t^T (scale * q_t)
 *
 * Sources:
 *   - "Understanding Kimi Delta Attention" (A. Flores), section "Learning what
 *     to forget", box "KDA: retain, predict, correct" (the three state lines and
 *     the order: decay first, then predict from the decayed state, then
 *     correct), and the closing sentence of that section (the query reads the
 *     UPDATED state).
 *   - "Demystifying Kimi Delta Attention" (J. Dborin), section "The Complexity
 *     of Modern Linear Attention", first display (same recurrence in bra-ket
 *     form, with the d_k^{-1/2} query scale in the read).  That page writes the
 *     state as V x K (the transpose); the numbers are identical.
 *
 * The input g is the PER-TOKEN log-decay (not cumulative).  Nothing is
 * normalised, clamped or validated here: the oracle evaluates the definition
 * on whatever it is given.
 *
 * Parallelism: OpenMP over independent (sequence, head, column-block) units.
 * Column c of S and of o depends only on column c of v and of S_0 (every
 * operation above acts on columns independently), so the split changes no
 * arithmetic: each element sees exactly the same sequence of fp64 operations.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of one head on state columns [c0, c1).  S is d_k x d_v row-major
 * (row r = key channel r).  tmp holds d_v doubles of scratch. */
static void kda_oracle_token(int dk, int dv, int c0, int c1, double *S,
                             const double *q, const double *k, const double *v,
                             const double *g, double beta, double scale,
                             double *o, double *tmp)
{
    int r, c;
    /* retain: scale row r of the state by a[r] = exp(g[r]) */
    for (r = 0; r < dk; ++r) {
        double a = exp(g[r]);
        double *row = S + (size_t)r * dv;
        for (c = c0; c < c1; ++c) row[c] *= a;
    }
    /* predict: v_hat = S_bar^T k (kept in tmp) */
    for (c = c0; c < c1; ++c) tmp[c] = 0.0;
    for (r = 0; r < dk; ++r) {
        const double *row = S + (size_t)r * dv;
        for (c = c0; c < c1; ++c) tmp[c] += row[c] * k[r];
    }
    /* correct: S <- S_bar + beta k (v - v_hat)^T  (tmp becomes the error) */
    for (c = c0; c < c1; ++c) tmp[c] = v[c] - tmp[c];
    for (r = 0; r < dk; ++r) {
        double *row = S + (size_t)r * dv;
        double bk = beta * k[r];
        for (c = c0; c < c1; ++c) row[c] += bk * tmp[c];
    }
    /* read the updated state: o = S^T (scale q) */
    for (c = c0; c < c1; ++c) o[c] = 0.0;
    for (r = 0; r < dk; ++r) {
        const double *row = S + (size_t)r * dv;
        double sq = scale * q[r];
        for (c = c0; c < c1; ++c) o[c] += row[c] * sq;
    }
}

/*
 * Prefill over packed sequences.
 *   cu_seqlens [n_seqs+1], non-decreasing, cu_seqlens[0] == 0; sequence n owns
 *              packed tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *   q, k, g    [T_total, H, d_k]      v, o  [T_total, H, d_v]      beta [T_total, H]
 *   s0         [n_seqs, H, d_k, d_v]  or NULL (zero initial state)
 *   s_final    [n_seqs, H, d_k, d_v]  (always written; a zero-length sequence
 *              returns its initial state)
 *   col_block  columns per parallel unit (<= 0: all d_v columns in one unit)
 *   n_threads  OpenMP threads (<= 0: the runtime default)
 * Returns 0 on success, -1 on a bad argument (nothing is written then).
 */
int kda_oracle_prefill(int32_t n_seqs, const int64_t *cu_seqlens, int32_t H,
                       int32_t dk, int32_t dv, const double *q, const double *k,
                       const double *v, const double *g, const double *beta,
                       double scale, const double *s0, double *o,
                       double *s_final, int32_t col_block, int32_t n_threads)
{
    int64_t n_units, u;
    int32_t n_cb, n;
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || !s_final) return -1;
    if (cu_seqlens[0] != 0) return -1;
    for (n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    if (col_block <= 0 || col_block > dv) col_block = dv;
    n_cb = (dv + col_block - 1) / col_block;
    n_units = (int64_t)n_seqs * H * n_cb;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel
    {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (u = 0; u < n_units; ++u) {
            int32_t cb = (int32_t)(u % n_cb);
            int32_t h = (int32_t)((u / n_cb) % H);
            int32_t s = (int32_t)(u / ((int64_t)n_cb * H));
            int c0 = cb * col_block, c1 = c0 + col_block;
            int64_t t;
            size_t sd = (size_t)dk * dv;
            double *S = s_final + ((size_t)s * H + h) * sd;
            int r, c;
            if (c1 > dv) c1 = dv;
            for (r = 0; r < dk; ++r)
                for (c = c0; c < c1; ++c)
                    S[(size_t)r * dv + c] = s0 ? s0[((size_t)s * H + h) * sd + (size_t)r * dv + c] : 0.0;
            for (t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
                size_t th = (size_t)t * H + h;
                kda_oracle_token(dk, dv, c0, c1, S, q + th * dk, k + th * dk,
                                 v + th * dv, g + th * dk, beta[th], scale,
                                 o + th * dv, tmp);
            }
        }
        free(tmp);
    }
    return 0;
}

/*
 * One decode step for n_sessions x H independent (session, head) pairs: the
 * same token body applied once, with the state updated in place.
 *   q, k, g [N, H, d_k]   v, o [N, H, d_v]   beta [N, H]   state [N, H, d_k, d_v]
 */
int kda_oracle_decode_step(int32_t n_sessions, int32_t H, int32_t dk, int32_t dv,
                           const double *q, const double *k, const double *v,
                           const double *g, const double *beta, double scale,
                           double *state, double *o, int32_t n_threads)
{
    int64_t n_units, u;
    if (n_sessions < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (n_sessions > 0 && (!q || !k || !v || !g || !beta || !state || !o)) return -1;
    n_units = (int64_t)n_sessions * H;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (u = 0; u < n_units; ++u) {
            kda_oracle_token(dk, dv, 0, dv, state + (size_t)u * dk * dv,
                             q + (size_t)u * dk, k + (size_t)u * dk,
                             v + (size_t)u * dv, g + (size_t)u * dk, beta[u],
                             scale, o + (size_t)u * dv, tmp);
        }
        free(tmp);
    }
    return 0;
}

/* Threads an OpenMP parallel region would use (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

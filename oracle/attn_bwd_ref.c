/*
 * attn_bwd_ref.c -- double-precision reference for the gradients of exact scaled
 * dot-product attention (the backward pass).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * links, loads or calls it, and it shares no code, header or constant with that
 * path.
 *
 * The forward is the plain definition (row softmax of the scaled, masked scores
 * times V).  With p_ij its probabilities and dO the upstream gradient of O, the
 * chain rule through that definition gives
 *
 *   dV_j  = sum_i p_ij dO_i                      (O = P V)
 *   dp_ij = dO_i . v_j
 *   D_i   = sum_j p_ij dp_ij                     (row term of the softmax Jacobian)
 *   ds_ij = p_ij (dp_ij - D_i)                   (gradient of the scaled score)
 *   dQ_i  = scale sum_j ds_ij k_j
 *   dK_j  = scale sum_i ds_ij q_i
 *
 * Source: "FlashAttention 怎么做? online softmax 怎么更新?", section
 * "Recomputation": the backward needs P but keeps only O and one logsumexp per
 * row, and rebuilds S and P from the inputs.  The pages give no gradient
 * formulas; the ones above are the derivative of the forward definition written
 * out (the reading recorded with the others in the design notes).  Nothing is
 * tiled: every row's whole score row is rebuilt, and every key's gradient is a
 * plain sum over the rows that see it.  Parallelism is only across independent
 * items.
 *
 * Visibility: key j is visible to query i iff (wl < 0 or j >= i - wl) and
 * (wr < 0 or j <= i + wr), the window of the window forward reference; causal
 * (top-left, j <= i) is (-1, 0) and full attention (-1, -1).  A row that sees no
 * key has O = 0, contributes nothing and gets dq = 0.
 *
 * oracle_attention_bwd_window_f64 / oracle_attention_bwd_f64 (causal 0 or 1)
 *   q, dout [B, H, Lq, d], k, v [B, H, Lk, d]   row-major, double
 *   rows  NULL: dq for every query row; else int64 [B*H, nrows] query indices
 *   keys  NULL: dk, dv for every key;   else int64 [B*H, nkeys] key indices
 *   dq [B*H, nr, d], dk and dv [B*H, nk, d] (nr = Lq or nrows, nk = Lk or nkeys)
 * Returns ORACLE_OK, ORACLE_ERR_ARG or ORACLE_ERR_NOMEM.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* Keys [*lo, *hi) visible to query i. */
static void keys_of_row(int i, int Lk, int wl, int wr, int *lo, int *hi)
{
    int64_t a = 0, b = Lk;
    if (wl >= 0 && (int64_t)i - wl > a) a = (int64_t)i - wl;
    if (wr >= 0 && (int64_t)i + wr + 1 < b) b = (int64_t)i + wr + 1;
    *lo = (int)a;
    *hi = (int)(b > a ? b : a);
}

/* Queries [*lo, *hi) that see key j (the same predicate solved for i). */
static void rows_of_key(int j, int Lq, int wl, int wr, int *lo, int *hi)
{
    int64_t a = 0, b = Lq;
    if (wr >= 0 && (int64_t)j - wr > a) a = (int64_t)j - wr;
    if (wl >= 0 && (int64_t)j + wl + 1 < b) b = (int64_t)j + wl + 1;
    *lo = (int)a;
    *hi = (int)(b > a ? b : a);
}

int oracle_attention_bwd_window_f64(const double *q, const double *k, const double *v, const double *dout,
                                    int B, int H, int Lq, int Lk, int d, double scale, int wl, int wr,
                                    const int64_t *rows, int nrows, const int64_t *keys, int nkeys,
                                    double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || d <= 0) return ORACLE_ERR_ARG;
    const int nr = rows ? nrows : Lq;
    const int nk = keys ? nkeys : Lk;
    if (nr <= 0 || nk <= 0) return ORACLE_ERR_ARG;
    if (rows)
        for (int64_t x = 0; x < (int64_t)B * H * nr; ++x)
            if (rows[x] < 0 || rows[x] >= Lq) return ORACLE_ERR_ARG;
    if (keys)
        for (int64_t x = 0; x < (int64_t)B * H * nk; ++x)
            if (keys[x] < 0 || keys[x] >= Lk) return ORACLE_ERR_ARG;
    const int64_t BH = (int64_t)B * H;
    /* per-row logsumexp and D_i of every row of every head */
    double *lse = (double *)malloc(sizeof(double) * (size_t)(BH * Lq));
    double *Drow = (double *)malloc(sizeof(double) * (size_t)(BH * Lq));
    /* row position -> index in `rows` (-1: no dq wanted) */
    int *want = (int *)malloc(sizeof(int) * (size_t)(BH * Lq));
    if (!lse || !Drow || !want) {
        free(lse); free(Drow); free(want);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t x = 0; x < BH * Lq; ++x)
        want[x] = rows ? -1 : (int)(x % Lq);
    if (rows)
        for (int64_t bh = 0; bh < BH; ++bh)
            for (int r = 0; r < nr; ++r)
                want[bh * Lq + rows[bh * nr + r]] = r;
    int bad = 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Lk);
        double *dp = (double *)malloc(sizeof(double) * (size_t)Lk);
        if (!s || !dp) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
        /* 1. every row: probabilities, D_i, lse_i, and dq where wanted */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t it = 0; it < BH * Lq; ++it) {
            if (!s || !dp) continue;
            const int64_t bh = it / Lq;
            const int i = (int)(it % Lq);
            const double *qi = q + ((size_t)bh * Lq + i) * d;
            const double *doi = dout + ((size_t)bh * Lq + i) * d;
            const double *Kb = k + (size_t)bh * Lk * d;
            const double *Vb = v + (size_t)bh * Lk * d;
            int lo, hi;
            keys_of_row(i, Lk, wl, wr, &lo, &hi);
            for (int j = lo; j < hi; ++j) {
                double dot = 0.0, dd = 0.0;
                for (int t = 0; t < d; ++t) {
                    dot += qi[t] * Kb[(size_t)j * d + t];
                    dd += doi[t] * Vb[(size_t)j * d + t];
                }
                s[j - lo] = scale * dot;
                dp[j - lo] = dd;
            }
            double m = -INFINITY;
            for (int j = lo; j < hi; ++j)
                if (s[j - lo] > m) m = s[j - lo];
            double l = 0.0;
            for (int j = lo; j < hi; ++j)
                l += exp(s[j - lo] - m);
            double Di = 0.0;
            for (int j = lo; j < hi; ++j)
                Di += exp(s[j - lo] - m) / l * dp[j - lo];
            lse[it] = hi > lo ? m + log(l) : -INFINITY;
            Drow[it] = Di;
            const int r = want[it];
            if (r >= 0) {
                double *dqi = dq + ((size_t)bh * nr + r) * d;
                for (int t = 0; t < d; ++t)
                    dqi[t] = 0.0;
                for (int j = lo; j < hi; ++j) {
                    const double p = exp(s[j - lo] - m) / l;
                    const double ds = p * (dp[j - lo] - Di);
                    for (int t = 0; t < d; ++t)
                        dqi[t] += scale * ds * Kb[(size_t)j * d + t];
                }
            }
        }
        /* 2. every wanted key: sums over the rows that see it */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t it = 0; it < BH * nk; ++it) {
            const int64_t bh = it / nk;
            const int x = (int)(it % nk);
            const int j = keys ? (int)keys[bh * nk + x] : x;
            const double *kj = k + ((size_t)bh * Lk + j) * d;
            const double *vj = v + ((size_t)bh * Lk + j) * d;
            double *dkj = dk + (size_t)it * d;
            double *dvj = dv + (size_t)it * d;
            for (int t = 0; t < d; ++t) {
                dkj[t] = 0.0;
                dvj[t] = 0.0;
            }
            int ilo, ihi;
            rows_of_key(j, Lq, wl, wr, &ilo, &ihi);
            for (int i = ilo; i < ihi; ++i) {
                const double *qi = q + ((size_t)bh * Lq + i) * d;
                const double *doi = dout + ((size_t)bh * Lq + i) * d;
                double dot = 0.0, dd = 0.0;
                for (int t = 0; t < d; ++t) {
                    dot += qi[t] * kj[t];
                    dd += doi[t] * vj[t];
                }
                const double p = exp(scale * dot - lse[bh * Lq + i]);
                const double ds = p * (dd - Drow[bh * Lq + i]);
                for (int t = 0; t < d; ++t) {
                    dkj[t] += scale * ds * qi[t];
                    dvj[t] += p * doi[t];
                }
            }
        }
        free(s);
        free(dp);
    }
    free(lse);
    free(Drow);
    free(want);
    return bad ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

int oracle_attention_bwd_f64(const double *q, const double *k, const double *v, const double *dout,
                             int B, int H, int Lq, int Lk, int d, double scale, int causal,
                             const int64_t *rows, int nrows, const int64_t *keys, int nkeys,
                             double *dq, double *dk, double *dv, int nthreads)
{
    if (causal != 0 && causal != 1) return ORACLE_ERR_ARG;
    return oracle_attention_bwd_window_f64(q, k, v, dout, B, H, Lq, Lk, d, scale, -1, causal ? 0 : -1,
                                           rows, nrows, keys, nkeys, dq, dk, dv, nthreads);
}

/*
 * attn_window_ref.c -- double-precision reference for exact attention restricted
 * to a window of keys around each query (local / sliding-window attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * links, loads or calls it, and it shares no code, header or constant with that
 * path.
 *
 * Key j is visible to query i iff
 *     (wl < 0 or j >= i - wl)  and  (wr < 0 or j <= i + wr),   0 <= j < Lk,
 * so (wl, wr) = (-1, -1) is full attention and (-1, 0) the causal mask with
 * top-left alignment.  For each visible key the score is s_ij = scale q_i.k_j;
 * then the three-pass safe softmax (max, sum of exp(s - m), divide), O = P V and
 * lse = m + ln l, exactly as the full-attention reference.  A row that sees no
 * key gets O = 0 and lse = -inf.
 *
 * Source: "Flash Attention 全解析（上）：从 V1、V2 到 Flash Decoding 的演进与思想",
 * section 5.3 names sliding-window attention as the variant the family goes on to
 * support; the pages give no formula, so the window above is the reading recorded
 * with the others in the design notes.  Definition of attention itself: section
 * 1.2 of the same page.  Nothing is tiled; parallel over (batch, head, row) only.
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

/* Visible key range [*lo, *hi) of query i. */
static void window_range(int i, int Lk, int wl, int wr, int *lo, int *hi)
{
    int64_t a = 0, b = Lk;
    if (wl >= 0 && (int64_t)i - wl > a) a = (int64_t)i - wl;
    if (wr >= 0 && (int64_t)i + wr + 1 < b) b = (int64_t)i + wr + 1;
    if (b < a) b = a;
    *lo = (int)a;
    *hi = (int)b;
}

/*
 * oracle_attention_window_f64
 *   q [B, H, Lq, d], k, v [B, H, Lk, d]  row-major, double
 *   wl, wr   window bounds as above (negative: unbounded on that side)
 *   rows     NULL: every query row; else int64 [B*H, nrows] query indices
 *   o [B*H, nr, d], lse [B*H, nr]  (nr = Lq or nrows)
 * Returns ORACLE_OK, ORACLE_ERR_ARG or ORACLE_ERR_NOMEM.
 */
int oracle_attention_window_f64(const double *q, const double *k, const double *v,
                                int B, int H, int Lq, int Lk, int d, double scale, int wl, int wr,
                                const int64_t *rows, int nrows, double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || d <= 0) return ORACLE_ERR_ARG;
    const int nr = rows ? nrows : Lq;
    if (nr <= 0) return ORACLE_ERR_ARG;
    if (rows)
        for (int64_t x = 0; x < (int64_t)B * H * nr; ++x)
            if (rows[x] < 0 || rows[x] >= Lq) return ORACLE_ERR_ARG;
    const int64_t items = (int64_t)B * H * nr;
    int bad = 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)Lk);
        if (!sc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t it = 0; it < items; ++it) {
            if (!sc) continue;
            const int64_t bh = it / nr;
            const int r = (int)(it % nr);
            const int i = rows ? (int)rows[bh * nr + r] : r;
            const double *query = q + ((size_t)bh * Lq + i) * d;
            double *out = o + (size_t)it * d;
            int lo, hi;
            window_range(i, Lk, wl, wr, &lo, &hi);
            for (int t = 0; t < d; ++t)
                out[t] = 0.0;
            if (hi == lo) {                       /* no visible key */
                lse[it] = -INFINITY;
                continue;
            }
            double mx = -INFINITY;
            for (int j = lo; j < hi; ++j) {
                const double *key = k + ((size_t)bh * Lk + j) * d;
                double dot = 0.0;
                for (int t = 0; t < d; ++t)
                    dot += query[t] * key[t];
                sc[j - lo] = scale * dot;
                if (sc[j - lo] > mx) mx = sc[j - lo];
            }
            double sum = 0.0;
            for (int j = lo; j < hi; ++j)
                sum += exp(sc[j - lo] - mx);
            for (int j = lo; j < hi; ++j) {
                const double w = exp(sc[j - lo] - mx) / sum;
                const double *val = v + ((size_t)bh * Lk + j) * d;
                for (int t = 0; t < d; ++t)
                    out[t] += w * val[t];
            }
            lse[it] = mx + log(sum);
        }
        free(sc);
    }
    return bad ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

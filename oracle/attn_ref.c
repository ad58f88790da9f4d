/*
 * attn_ref.c -- double-precision reference for exact scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the HIP
 * library and its Python binding) never links, loads or calls it, and it shares
 * no code, header or constant with that path.
 *
 * What it computes is the plain definition of attention, not the tiled method:
 *
 *   s_ij   = scale * sum_t q_it * k_jt        for every key j visible to query i
 *   m_i    = max_j s_ij                       (pass 1 of the safe softmax)
 *   l_i    = sum_j exp(s_ij - m_i)            (pass 2)
 *   p_ij   = exp(s_ij - m_i) / l_i            (pass 3)
 *   o_i    = sum_j p_ij * v_j                 (the P*V product)
 *   lse_i  = m_i + ln(l_i)                    (natural-log logsumexp of the scaled row)
 *
 * Sources: "Flash Attention 全解析（上）：从 V1、V2 到 Flash Decoding 的演进与思想",
 * section 1.2 (standard attention: S = QK^T, P = softmax(S), O = PV, and the
 * three-pass safe softmax: row max, sum of exponentials, divide);
 * "Triton内核实战：手写FlashAttention-2，优化长序列GPU内存瓶颈", section
 * "标准注意力为何是内存瓶颈" (same definition with the scaled dot product);
 * "FlashAttention 怎么做? online softmax 怎么更新?", section "必答点 /
 * FlashAttention-2 改了什么" (one logsumexp L = m + log l per row).
 *
 * Readings where the pages are silent (each is listed with the others in the
 * project's design notes):
 *   - causal visibility is top-left: key j is visible to query i iff j <= i;
 *   - scale multiplies the raw dot product before the max;
 *   - lse uses the natural logarithm of the scaled scores over visible keys.
 *
 * The whole score row is materialised (length <= Lk) -- nothing is tiled, fused
 * or reordered.  Parallelism is only across independent (batch, head, row) items.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of this reference (independent of the product library's codes). */
#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* One query row against the first `nvis` keys of one (batch, head). */
static void attend_one_row(const double *q, const double *K, const double *V,
                           int nvis, int d, double scale,
                           double *s /* scratch, >= nvis */, double *o, double *lse)
{
    /* scores of the visible keys */
    for (int j = 0; j < nvis; ++j) {
        double dot = 0.0;
        for (int t = 0; t < d; ++t)
            dot += q[t] * K[(size_t)j * d + t];
        s[j] = scale * dot;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int j = 0; j < nvis; ++j)
        if (s[j] > m) m = s[j];
    /* pass 2: sum of shifted exponentials */
    double l = 0.0;
    for (int j = 0; j < nvis; ++j)
        l += exp(s[j] - m);
    /* pass 3: probabilities, accumulated straight into O = P V */
    for (int t = 0; t < d; ++t)
        o[t] = 0.0;
    for (int j = 0; j < nvis; ++j) {
        const double p = exp(s[j] - m) / l;
        for (int t = 0; t < d; ++t)
            o[t] += p * V[(size_t)j * d + t];
    }
    *lse = m + log(l);
}

/*
 * oracle_attention_f64
 *   q   [B, H, Lq, d]  row-major, double (the exact values the device sees, widened)
 *   k,v [B, H, Lk, d]  row-major, double
 *   rows    NULL: every query row 0..Lq-1 of every (b, h) is computed, nrows ignored.
 *           else: an int64 array [B*H, nrows]; row r of (b,h) computes query index
 *                 rows[(b*H + h)*nrows + r] (must lie in [0, Lq)).
 *   o   [B*H, nr, d] double, nr = Lq or nrows;  lse [B*H, nr] double.
 *   nthreads  OpenMP threads (<= 0: the runtime's default).
 * Returns ORACLE_OK, or ORACLE_ERR_ARG for a bad size / pointer / row index.
 */
int oracle_attention_f64(const double *q, const double *k, const double *v,
                         int B, int H, int Lq, int Lk, int d, double scale, int causal,
                         const int64_t *rows, int nrows,
                         double *o, double *lse, int nthreads)
{
    if (!q || !k || !v || !o || !lse) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if (causal != 0 && causal != 1) return ORACLE_ERR_ARG;
    const int nr = rows ? nrows : Lq;
    if (nr <= 0) return ORACLE_ERR_ARG;
    if (rows) {
        for (int64_t x = 0; x < (int64_t)B * H * nr; ++x)
            if (rows[x] < 0 || rows[x] >= Lq) return ORACLE_ERR_ARG;
    }
    const int64_t items = (int64_t)B * H * nr;
    int bad = 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Lk);
        if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t it = 0; it < items; ++it) {
            if (!s) continue;
            const int64_t bh = it / nr;
            const int r = (int)(it % nr);
            const int i = rows ? (int)rows[bh * nr + r] : r;
            const double *qi = q + ((size_t)bh * Lq + i) * d;
            const double *Kb = k + (size_t)bh * Lk * d;
            const double *Vb = v + (size_t)bh * Lk * d;
            int nvis = Lk;
            if (causal && i + 1 < Lk) nvis = i + 1; /* keys 0..i */
            attend_one_row(qi, Kb, Vb, nvis, d, scale, s,
                           o + (size_t)it * d, lse + it);
        }
        free(s);
    }
    return bad ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * attn_dropout_ref.c -- double-precision reference for exact attention with
 * dropout on the attention probabilities (forward and gradients).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * links, loads or calls it, and it shares no code, header or constant with that
 * path.
 *
 * Dropout is the optional step the pages list among the operations fused into
 * one pass over a score block ("Flash Attention 全解析（上）", section 2.1.2: mask,
 * softmax, dropout, then the product with V); they give no formula or random
 * number generator.  Readings (recorded with the others in the design notes):
 *
 *   keep mask   z_ij = [u_ij < t], t = round(256 (1 - p)) in 1..256, where the byte
 *               u_ij comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 *               random numbers: as easy as 1, 2, 3", SC'11): counter
 *               (j / 4, i / 4, b H + h, offset), key (seed mod 2^32, seed / 2^32),
 *               output word i % 4, byte j % 4 (least significant first).
 *   scale       a kept probability is multiplied by 256 / t = 1 / (1 - p_eff),
 *               p_eff = 1 - t / 256, so E[z scale] = 1.
 *   forward     A_ij = P_ij z_ij 256 / t, O = A V; the logsumexp is that of the
 *               scores without dropout (the softmax statistics do not change).
 *   gradients   dV = A^T dO, dA = dO V^T, dP = dA z 256 / t, D_i = sum_j A_ij dA_ij
 *               (= dO_i . O_i), dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *
 * Everything else is the plain definition (visible keys, three-pass softmax,
 * fp64), causal visibility top-left.  Nothing is tiled.
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

/* Philox4x32-10 of the SC'11 paper: ten rounds of two 32x32->64-bit products
 * with the multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped by the Weyl
 * constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The dropout byte of element (i, j) of head bh. */
static uint32_t dropout_byte(int64_t bh, int i, int j, uint64_t seed, uint32_t offset)
{
    const uint32_t ctr[4] = {(uint32_t)(j / 4), (uint32_t)(i / 4), (uint32_t)bh, offset};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    return (w[i % 4] >> (8 * (j % 4))) & 0xFFu;
}

/* The keep mask of a whole [B*H, Lq, Lk] block as bytes (1 keep, 0 drop). */
int oracle_dropout_mask(int B, int H, int Lq, int Lk, uint64_t seed, uint32_t offset, int t, uint8_t *mask)
{
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || t < 1 || t > 256 || !mask) return ORACLE_ERR_ARG;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int i = 0; i < Lq; ++i)
            for (int j = 0; j < Lk; ++j)
                mask[((size_t)bh * Lq + i) * Lk + j] = dropout_byte(bh, i, j, seed, offset) < (uint32_t)t;
    return ORACLE_OK;
}

/*
 * oracle_attention_dropout_f64: forward (o, lse) and, when dout != NULL, the
 * gradients (dq, dk, dv) of attention with dropout, for every row and key.
 *   q, dout [B, H, Lq, d], k, v [B, H, Lk, d]; o [B, H, Lq, d], lse [B, H, Lq];
 *   dq [B, H, Lq, d], dk, dv [B, H, Lk, d]  (all double, row-major)
 *   t      keep threshold, 1..256 (keep probability t / 256)
 */
int oracle_attention_dropout_f64(const double *q, const double *k, const double *v, const double *dout,
                                 int B, int H, int Lq, int Lk, int d, double scale, int causal,
                                 uint64_t seed, uint32_t offset, int t,
                                 double *o, double *lse, double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !o || !lse) return ORACLE_ERR_ARG;
    if (dout && (!dq || !dk || !dv)) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if ((causal != 0 && causal != 1) || t < 1 || t > 256) return ORACLE_ERR_ARG;
    const int64_t BH = (int64_t)B * H;
    const double keep_scale = 256.0 / t;
    /* per row: probabilities P and the dropped, rescaled A of its visible keys,
       D_i; kept for the key pass of the gradients */
    double *Prow = (double *)malloc(sizeof(double) * (size_t)(BH * Lq) * Lk);
    double *Drow = (double *)malloc(sizeof(double) * (size_t)(BH * Lq));
    if (!Prow || !Drow) {
        free(Prow); free(Drow);
        return ORACLE_ERR_NOMEM;
    }

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
#endif
    for (int64_t it = 0; it < BH * Lq; ++it) {
        const int64_t bh = it / Lq;
        const int i = (int)(it % Lq);
        const double *qi = q + (size_t)it * d;
        double *P = Prow + (size_t)it * Lk;
        const int nvis = (causal && i + 1 < Lk) ? i + 1 : Lk;
        double mx = -INFINITY;
        for (int j = 0; j < nvis; ++j) {
            const double *kj = k + ((size_t)bh * Lk + j) * d;
            double dot = 0.0;
            for (int x = 0; x < d; ++x)
                dot += qi[x] * kj[x];
            P[j] = scale * dot;
            if (P[j] > mx) mx = P[j];
        }
        double l = 0.0;
        for (int j = 0; j < nvis; ++j)
            l += exp(P[j] - mx);
        for (int j = 0; j < nvis; ++j)
            P[j] = exp(P[j] - mx) / l;
        for (int j = nvis; j < Lk; ++j)
            P[j] = 0.0;
        lse[it] = mx + log(l);
        double *oi = o + (size_t)it * d;
        for (int x = 0; x < d; ++x)
            oi[x] = 0.0;
        double Di = 0.0;
        const double *doi = dout ? dout + (size_t)it * d : NULL;
        for (int j = 0; j < nvis; ++j) {
            const double a = dropout_byte(bh, i, j, seed, offset) < (uint32_t)t ? P[j] * keep_scale : 0.0;
            const double *vj = v + ((size_t)bh * Lk + j) * d;
            for (int x = 0; x < d; ++x)
                oi[x] += a * vj[x];
            if (doi) {
                double da = 0.0;
                for (int x = 0; x < d; ++x)
                    da += doi[x] * vj[x];
                Di += a * da;
            }
        }
        Drow[it] = Di;
        if (doi) {                                   /* dq of this row */
            double *dqi = dq + (size_t)it * d;
            for (int x = 0; x < d; ++x)
                dqi[x] = 0.0;
            for (int j = 0; j < nvis; ++j) {
                const double *vj = v + ((size_t)bh * Lk + j) * d;
                const double *kj = k + ((size_t)bh * Lk + j) * d;
                double da = 0.0;
                for (int x = 0; x < d; ++x)
                    da += doi[x] * vj[x];
                const double dp = dropout_byte(bh, i, j, seed, offset) < (uint32_t)t ? da * keep_scale : 0.0;
                const double ds = P[j] * (dp - Di);
                for (int x = 0; x < d; ++x)
                    dqi[x] += scale * ds * kj[x];
            }
        }
    }
    if (dout) {
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
#endif
        for (int64_t it = 0; it < BH * Lk; ++it) {       /* dk, dv of every key */
            const int64_t bh = it / Lk;
            const int j = (int)(it % Lk);
            const double *vj = v + (size_t)it * d;
            double *dkj = dk + (size_t)it * d;
            double *dvj = dv + (size_t)it * d;
            for (int x = 0; x < d; ++x) {
                dkj[x] = 0.0;
                dvj[x] = 0.0;
            }
            for (int i = causal ? j : 0; i < Lq; ++i) {
                const double p = Prow[((size_t)bh * Lq + i) * Lk + j];
                const int keep = dropout_byte(bh, i, j, seed, offset) < (uint32_t)t;
                const double a = keep ? p * keep_scale : 0.0;
                const double *qi = q + ((size_t)bh * Lq + i) * d;
                const double *doi = dout + ((size_t)bh * Lq + i) * d;
                double da = 0.0;
                for (int x = 0; x < d; ++x)
                    da += doi[x] * vj[x];
                const double dp = keep ? da * keep_scale : 0.0;
                const double ds = p * (dp - Drow[bh * Lq + i]);
                for (int x = 0; x < d; ++x) {
                    dvj[x] += a * doi[x];
                    dkj[x] += scale * ds * qi[x];
                }
            }
        }
    }
    free(Prow);
    free(Drow);
    return ORACLE_OK;
}

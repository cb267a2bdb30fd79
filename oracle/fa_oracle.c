/*
 * fa_oracle.c -- plain fp64 CPU attention oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline of the benchmark load this library.  It shares no code, header or
 * table with the GPU path.
 *
 * What it computes (exact scaled-dot-product attention, "FlashAttention'ı
 * Anlamak Bölüm 1", section 0.2 "Notasyon", the score/output equations with
 * the optional mask/bias term taken as zero):
 *
 *     s_ij  = sigma * sum_c q_ic k_jc          (sigma = the caller's float scale)
 *     m_i   = max_j s_ij
 *     e_ij  = exp(s_ij - m_i)
 *     l_i   = sum_j e_ij
 *     O_ic  = (sum_j e_ij v_jc) / l_i
 *     LSE_i = m_i + ln(l_i)
 *
 * The same section states the method is exact (not low-rank or sparse): only
 * the floating-point order may differ, so the oracle is the definition itself.
 * It follows the two-pass reading of the unfused algorithm in section 0.1
 * ("Bu Rehber Nasıl Okunmalı?": compute S, then P, then O), one query row at a
 * time instead of materialising the N x N matrices.  Subtracting the row max
 * before exp is an identity (softmax is shift invariant) that keeps exp finite.
 *
 * Inputs are bf16 bit patterns (uint16), [B, H, N, d] row-major, widened
 * exactly to fp64.  All sums are sequential fp64.  Nothing is rounded to bf16.
 * OpenMP distributes whole rows over threads; each row's arithmetic order is
 * fixed, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One query row against one head's K [Nk, d] and V [Nk, dv]. */
static void attend_one_row(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                           int64_t Nk, int64_t d, int64_t dv, double sigma,
                           double *s, double *o, double *lse)
{
    for (int64_t j = 0; j < Nk; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += widen_bf16(q[c]) * widen_bf16(K[j * d + c]);
        s[j] = sigma * dot;
    }
    double m = s[0];
    for (int64_t j = 1; j < Nk; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < Nk; ++j)
        for (int64_t c = 0; c < dv; ++c)
            o[c] += s[j] * widen_bf16(V[j * dv + c]);
    for (int64_t c = 0; c < dv; ++c) o[c] /= l;
    *lse = m + log(l);
}

/* Returns 0 on success, -1 on bad arguments, -2 when scratch allocation fails. */
static int attend_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                       float scale, const int64_t *rows, int64_t n_rows,
                       double *O, double *LSE)
{
    if (!Q || !K || !V || !O || !LSE) return -1;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || d < 1 || dv < 1 || n_rows < 0) return -1;
    const double sigma = (double)scale;
    const int64_t total = B * H * Nq;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            const int64_t flat = rows ? rows[r] : r;
            if (flat < 0 || flat >= total) {
#pragma omp atomic write
                failed = -1;
                continue;
            }
            const int64_t bh = flat / Nq;
            attend_one_row(Q + flat * d, K + bh * Nk * d, V + bh * Nk * dv,
                           Nk, d, dv, sigma, s, O + r * dv, LSE + r);
        }
        free(s);
    }
    return failed;
}

/* Full attention: O [B,H,Nq,dv] fp64, LSE [B,H,Nq] fp64 (natural log). */
int oracle_attn_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                     float scale, double *O, double *LSE)
{
    return attend_rows(Q, K, V, B, H, Nq, Nk, d, dv, scale, NULL, B * H * Nq, O, LSE);
}

/* Selected rows: rows[r] is a flat index into [B*H*Nq]; O is [n_rows, dv]. */
int oracle_attn_rows_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                          float scale, const int64_t *rows, int64_t n_rows,
                          double *O, double *LSE)
{
    if (!rows && n_rows > 0) return -1;
    return attend_rows(Q, K, V, B, H, Nq, Nk, d, dv, scale, rows, n_rows, O, LSE);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

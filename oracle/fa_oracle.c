/*
 * fa_oracle.c -- plain fp64 CPU attention oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline of the benchmark load this library.  It shares no code, header or
 * table with the GPU path.
 *
 * What it computes (exact scaled-dot-product attention, "FlashAttention'ı
 * Anlamak Bölüm 1", section 0.2 "Notasyon", the score/output equations; the
 * optional mask/bias term is described further down):
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
 * The same section's optional mask/bias term B is supported as an fp32
 * additive bias (s_ij += B_ij, broadcast over batch and heads through zero
 * strides) and as a causal mask, which hides key j from query i when
 * j > i + (Nk - Nq) (the diagonal aligned to the last query and key).  A row
 * that sees no key at all (causal with Nq > Nk, or every bias entry -inf) has
 * no softmax; the oracle reports O = 0 and LSE = -inf for it.
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

/* One query row against the first n_vis keys of one head's K [Nk, d] and
 * V [Nk, dv]; bias_row (may be NULL) holds the row's additive bias. */
static void attend_one_row(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                           int64_t n_vis, int64_t d, int64_t dv, double sigma,
                           const float *bias_row, double *s, double *o, double *lse)
{
    for (int64_t j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += widen_bf16(q[c]) * widen_bf16(K[j * d + c]);
        s[j] = sigma * dot;
        if (bias_row) s[j] += (double)bias_row[j];
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j)
        if (s[j] > m) m = s[j];
    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    if (m == -INFINITY) {  /* no visible key */
        *lse = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t j = 0; j < n_vis; ++j)
        for (int64_t c = 0; c < dv; ++c)
            o[c] += s[j] * widen_bf16(V[j * dv + c]);
    for (int64_t c = 0; c < dv; ++c) o[c] /= l;
    *lse = m + log(l);
}

/* Returns 0 on success, -1 on bad arguments, -2 when scratch allocation fails. */
static int attend_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                       float scale, int causal, const float *bias,
                       int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                       const int64_t *rows, int64_t n_rows, double *O, double *LSE)
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
            const int64_t i = flat - bh * Nq;
            int64_t n_vis = Nk;
            if (causal) {
                n_vis = i + (Nk - Nq) + 1;
                if (n_vis < 0) n_vis = 0;
                if (n_vis > Nk) n_vis = Nk;
            }
            const float *bias_row = bias ? bias + (bh / H) * bias_sb + (bh % H) * bias_sh + i * bias_sq : NULL;
            attend_one_row(Q + flat * d, K + bh * Nk * d, V + bh * Nk * dv, n_vis, d, dv, sigma,
                           bias_row, s, O + r * dv, LSE + r);
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
    return attend_rows(Q, K, V, B, H, Nq, Nk, d, dv, scale, 0, NULL, 0, 0, 0, NULL, B * H * Nq, O, LSE);
}

/* Selected rows: rows[r] is a flat index into [B*H*Nq]; O is [n_rows, dv]. */
int oracle_attn_rows_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                          float scale, const int64_t *rows, int64_t n_rows,
                          double *O, double *LSE)
{
    if (!rows && n_rows > 0) return -1;
    return attend_rows(Q, K, V, B, H, Nq, Nk, d, dv, scale, 0, NULL, 0, 0, 0, rows, n_rows, O, LSE);
}

/* With the mask/bias term: causal (0/1) and an optional fp32 bias addressed as
 * bias[b*bias_sb + h*bias_sh + i*bias_sq + j].  rows == NULL means all rows in
 * order (then n_rows must be B*H*Nq). */
int oracle_attn_masked_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                            float scale, int causal, const float *bias,
                            int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                            const int64_t *rows, int64_t n_rows, double *O, double *LSE)
{
    if (!rows && n_rows != B * H * Nq) return -1;
    return attend_rows(Q, K, V, B, H, Nq, Nk, d, dv, scale, causal != 0, bias,
                       bias_sb, bias_sh, bias_sq, rows, n_rows, O, LSE);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

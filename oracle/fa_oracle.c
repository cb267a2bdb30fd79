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

/* Keys visible to query row i: all Nk, or with the causal mask those with
 * j <= i + (Nk - Nq) (the diagonal aligned to the last query and key). */
static int64_t visible_keys(int causal, int64_t i, int64_t Nq, int64_t Nk)
{
    if (!causal) return Nk;
    int64_t n_vis = i + (Nk - Nq) + 1;
    if (n_vis < 0) n_vis = 0;
    if (n_vis > Nk) n_vis = Nk;
    return n_vis;
}

/* Bias row of query i of head bh (NULL when there is no bias). */
static const float *bias_row_of(const float *bias, int64_t bh, int64_t H, int64_t i,
                                int64_t sb, int64_t sh, int64_t sq)
{
    return bias ? bias + (bh / H) * sb + (bh % H) * sh + i * sq : NULL;
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
            const int64_t n_vis = visible_keys(causal, i, Nq, Nk);
            const float *bias_row = bias_row_of(bias, bh, H, i, bias_sb, bias_sh, bias_sq);
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

/* ------------------------------------------------------------------------
 * Backward pass (gradients of a scalar loss L through O, given dO = dL/dO).
 *
 * The pages motivate storing only the softmax statistics and recomputing
 * the attention matrix in the backward pass ("FlashAttention'ı Anlamak
 * Bölüm 1", section 0 "Giriş": recomputation, forward and backward passes).
 * The gradients themselves follow from the score and output equations of
 * section 0.2 by the chain rule, per query row i of one head:
 *
 *     P_ij  = softmax_j(s_ij),            s_ij = sigma * q_i . k_j (+ bias_ij)
 *     dV_j += P_ij dO_i                   (O_i = sum_j P_ij V_j)
 *     dP_ij = dO_i . V_j
 *     D_i   = sum_j P_ij dP_ij            (the softmax Jacobian's rank-one term)
 *     dS_ij = P_ij (dP_ij - D_i)          (dL/ds_ij)
 *     dQ_i  = sigma * sum_j dS_ij K_j
 *     dK_j += sigma * dS_ij Q_i
 *
 * Hidden keys (causal mask, -inf bias) have P_ij = 0 and contribute nothing;
 * a row that sees no key contributes nothing and gets dQ_i = 0.  Everything
 * is fp64 from the bf16 bits of Q, K, V and dO; no value is rounded.
 * ------------------------------------------------------------------------ */

/* Softmax probabilities of one row into p[0..n_vis) (NULL bias_row: none).
 * Returns 0 when the row sees no key (then p is untouched), else 1. */
static int row_probs(const uint16_t *q, const uint16_t *K, int64_t n_vis, int64_t d, double sigma,
                     const float *bias_row, double *p, double *lse)
{
    for (int64_t j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += widen_bf16(q[c]) * widen_bf16(K[j * d + c]);
        p[j] = sigma * dot;
        if (bias_row) p[j] += (double)bias_row[j];
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j)
        if (p[j] > m) m = p[j];
    if (m == -INFINITY) {
        if (lse) *lse = -INFINITY;
        return 0;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;
    if (lse) *lse = m + log(l);
    return 1;
}

/* dP_ij = dO_i . V_j into dp[0..n_vis); returns D_i = sum_j P_ij dP_ij. */
static double row_dp(const uint16_t *dOi, const uint16_t *V, int64_t n_vis, int64_t dv,
                     const double *p, double *dp)
{
    double Di = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < dv; ++c)
            dot += widen_bf16(dOi[c]) * widen_bf16(V[j * dv + c]);
        dp[j] = dot;
        Di += p[j] * dot;
    }
    return Di;
}

static int bwd_args_ok(const void *Q, const void *K, const void *V, const void *dO,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv)
{
    if (!Q || !K || !V || !dO) return 0;
    if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || d < 1 || dv < 1) return 0;
    return 1;
}

/* Full backward: dQ [B,H,Nq,d], dK [B,H,Nk,d], dV [B,H,Nk,dv] (fp64), plus
 * D and LSE [B,H,Nq].  Heads run in parallel; each head's rows run in order,
 * so the sums into dK and dV have a fixed order.  Returns 0, -1 (bad
 * arguments) or -2 (allocation failure). */
int oracle_attn_bwd_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *dO,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                         float scale, int causal, const float *bias,
                         int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                         double *dQ, double *dK, double *dV, double *D, double *LSE)
{
    if (!bwd_args_ok(Q, K, V, dO, B, H, Nq, Nk, d, dv) || !dQ || !dK || !dV || !D || !LSE) return -1;
    const double sigma = (double)scale;
    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)Nk * sizeof(double));
        double *dp = (double *)malloc((size_t)Nk * sizeof(double));
        if (!p || !dp) {
#pragma omp atomic write
            failed = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!p || !dp) continue;
            const uint16_t *Kh = K + bh * Nk * d, *Vh = V + bh * Nk * dv;
            double *dKh = dK + bh * Nk * d, *dVh = dV + bh * Nk * dv;
            for (int64_t t = 0; t < Nk * d; ++t) dKh[t] = 0.0;
            for (int64_t t = 0; t < Nk * dv; ++t) dVh[t] = 0.0;
            for (int64_t i = 0; i < Nq; ++i) {
                const int64_t row = bh * Nq + i;
                const uint16_t *qi = Q + row * d, *dOi = dO + row * dv;
                double *dQi = dQ + row * d;
                for (int64_t c = 0; c < d; ++c) dQi[c] = 0.0;
                const int64_t n_vis = visible_keys(causal, i, Nq, Nk);
                const float *bias_row = bias_row_of(bias, bh, H, i, bias_sb, bias_sh, bias_sq);
                if (!row_probs(qi, Kh, n_vis, d, sigma, bias_row, p, &LSE[row])) {
                    D[row] = 0.0;
                    continue;
                }
                const double Di = row_dp(dOi, Vh, n_vis, dv, p, dp);
                D[row] = Di;
                for (int64_t j = 0; j < n_vis; ++j) {
                    const double ds = p[j] * (dp[j] - Di);
                    for (int64_t c = 0; c < d; ++c) {
                        dQi[c] += sigma * ds * widen_bf16(Kh[j * d + c]);
                        dKh[j * d + c] += sigma * ds * widen_bf16(qi[c]);
                    }
                    for (int64_t c = 0; c < dv; ++c)
                        dVh[j * dv + c] += p[j] * widen_bf16(dOi[c]);
                }
            }
        }
        free(p);
        free(dp);
    }
    return failed;
}

/* dQ of selected query rows (flat indices into [B*H*Nq]): dQ [n_rows, d].
 * bias (may be NULL) as for oracle_attn_bwd_fp64. */
int oracle_attn_bwd_dq_rows_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *dO,
                                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                                 float scale, int causal, const float *bias,
                                 int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                                 const int64_t *rows, int64_t n_rows, double *dQ)
{
    if (!bwd_args_ok(Q, K, V, dO, B, H, Nq, Nk, d, dv) || !dQ || n_rows < 0 || (n_rows > 0 && !rows)) return -1;
    const double sigma = (double)scale;
    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)Nk * sizeof(double));
        double *dp = (double *)malloc((size_t)Nk * sizeof(double));
        if (!p || !dp) {
#pragma omp atomic write
            failed = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!p || !dp) continue;
            const int64_t flat = rows[r];
            double *dQi = dQ + r * d;
            for (int64_t c = 0; c < d; ++c) dQi[c] = 0.0;
            if (flat < 0 || flat >= B * H * Nq) {
#pragma omp atomic write
                failed = -1;
                continue;
            }
            const int64_t bh = flat / Nq, i = flat - bh * Nq;
            const uint16_t *Kh = K + bh * Nk * d, *Vh = V + bh * Nk * dv;
            const int64_t n_vis = visible_keys(causal, i, Nq, Nk);
            const float *bias_row = bias_row_of(bias, bh, H, i, bias_sb, bias_sh, bias_sq);
            if (!row_probs(Q + flat * d, Kh, n_vis, d, sigma, bias_row, p, NULL)) continue;
            const double Di = row_dp(dO + flat * dv, Vh, n_vis, dv, p, dp);
            for (int64_t j = 0; j < n_vis; ++j) {
                const double ds = p[j] * (dp[j] - Di);
                for (int64_t c = 0; c < d; ++c) dQi[c] += sigma * ds * widen_bf16(Kh[j * d + c]);
            }
        }
        free(p);
        free(dp);
    }
    return failed;
}

/* dK and dV of selected keys (flat indices into [B*H*Nk]): dK [n_keys, d],
 * dV [n_keys, dv].  Each key needs every query row's probabilities, so the
 * rows of each head that owns a selected key are visited in order and
 * scattered into the selected keys only. */
int oracle_attn_bwd_dkdv_keys_fp64(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *dO,
                                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                                   float scale, int causal, const float *bias,
                                   int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                                   const int64_t *keys, int64_t n_keys, double *dK, double *dV)
{
    if (!bwd_args_ok(Q, K, V, dO, B, H, Nq, Nk, d, dv) || !dK || !dV || n_keys < 0 || (n_keys > 0 && !keys))
        return -1;
    for (int64_t r = 0; r < n_keys; ++r)
        if (keys[r] < 0 || keys[r] >= B * H * Nk) return -1;
    const double sigma = (double)scale;
    for (int64_t t = 0; t < n_keys * d; ++t) dK[t] = 0.0;
    for (int64_t t = 0; t < n_keys * dv; ++t) dV[t] = 0.0;
    int failed = 0;
    /* one task per head; within it, query rows in order */
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)Nk * sizeof(double));
        double *dp = (double *)malloc((size_t)Nk * sizeof(double));
        if (!p || !dp) {
#pragma omp atomic write
            failed = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!p || !dp) continue;
            int any = 0;
            for (int64_t r = 0; r < n_keys; ++r) any |= keys[r] / Nk == bh;
            if (!any) continue;
            const uint16_t *Kh = K + bh * Nk * d, *Vh = V + bh * Nk * dv;
            for (int64_t i = 0; i < Nq; ++i) {
                const int64_t row = bh * Nq + i;
                const int64_t n_vis = visible_keys(causal, i, Nq, Nk);
                const float *bias_row = bias_row_of(bias, bh, H, i, bias_sb, bias_sh, bias_sq);
                if (!row_probs(Q + row * d, Kh, n_vis, d, sigma, bias_row, p, NULL)) continue;
                const double Di = row_dp(dO + row * dv, Vh, n_vis, dv, p, dp);
                for (int64_t r = 0; r < n_keys; ++r) {
                    if (keys[r] / Nk != bh) continue;
                    const int64_t j = keys[r] - bh * Nk;
                    if (j >= n_vis) continue;
                    const double ds = p[j] * (dp[j] - Di);
                    for (int64_t c = 0; c < d; ++c) dK[r * d + c] += sigma * ds * widen_bf16(Q[row * d + c]);
                    for (int64_t c = 0; c < dv; ++c) dV[r * dv + c] += p[j] * widen_bf16(dO[row * dv + c]);
                }
            }
        }
        free(p);
        free(dp);
    }
    return failed;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

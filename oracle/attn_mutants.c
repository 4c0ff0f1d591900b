/*
 * attn_mutants.c -- deliberately broken copies of the oracle (test
 * infrastructure for the pin tests only).
 *
 * THIS FILE IS TEST INFRASTRUCTURE.  Nothing here is the definition: the
 * definition is attend_row() and the backward in attn_oracle.c, which hold no
 * planted mistake.  This file restates the same computation once more with a
 * selectable deliberate mistake, so the pin tests can show that every
 * plausible mistake (a dropped term, a wrong sign or index, a transposed
 * operand) fails at least one pin.  It shares no code with attn_oracle.c and
 * none with the GPU path; single-threaded, tiny inputs only.
 *
 * Forward (page "flash-attn 实现 prefill 阶段", section 问题分析, the formula;
 * page "flash.cu", forward_kernel, the max-subtracted exponent):
 *   s_j = scale q_i.k_j, m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j,
 *   O_i = sum_j p_j v_j / l, LSE_i = m + ln l.
 * Backward (the calculus of the forward): dV_j = sum_i P_ij dO_i,
 *   dS_ij = P_ij (dO_i.v_j - D_i), D_i = sum_j P_ij dO_i.v_j,
 *   dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* forward mistakes (0 = none) */
enum {
    FM_NONE = 0,
    FM_NO_SCALE = 1,        /* scale never applied to the dot product     */
    FM_CAUSAL_STRICT = 2,   /* causal mask j < i instead of j <= i        */
    FM_K_TRANSPOSED = 3,    /* reads K as if stored [d, sk]               */
    FM_LSE_NO_MAX = 4,      /* LSE forgets to add the row max back        */
    FM_NO_NORMALISE = 5,    /* O is not divided by the row sum l          */
    FM_DROP_LAST_KEY = 6,   /* loop bound sk-1 instead of sk              */
    FM_EXP_SIGN = 7,        /* exp(m - s) instead of exp(s - m)           */
    FM_V_ROW_OFF = 8,       /* weights key j's probability onto V row j+1 */
    FM_MAX_LAST = 9         /* uses the last score instead of the max;
                               harmless in exact arithmetic, so this one
                               is caught only by overflow (a range pin)   */
};

/* backward mistakes (0 = none) */
enum {
    BM_NONE = 0,
    BM_NO_D = 1,          /* dS = P dP (the row term D forgotten)          */
    BM_DK_NO_SCALE = 2,   /* dK misses the scale                           */
    BM_DV_USES_DP = 3,    /* dV accumulates dP-weighted dO instead of P    */
    BM_DQ_USES_V = 4      /* dQ sums dS_ij v_j instead of dS_ij k_j        */
};

static int64_t m_keys(int64_t i, int64_t sk, int causal, int mut)
{
    int64_t lim = sk;
    if (causal) {
        const int64_t c = (mut == FM_CAUSAL_STRICT) ? i : i + 1;
        if (c < lim) lim = c;
    }
    if (mut == FM_DROP_LAST_KEY && lim > 1) lim -= 1;
    return lim;
}

static double m_dot(const double* a, const double* b, int64_t d, int64_t stride_b)
{
    double s = 0.0;
    for (int64_t x = 0; x < d; ++x) s += a[x] * b[x * stride_b];
    return s;
}

/* one row with forward mistake `mut`; p (scratch [sk]) receives the
 * normalised probabilities of the allowed keys; returns LSE_i */
static double m_row(const double* qi, const double* kh, const double* vh, int64_t i,
                     int64_t sk, int64_t d, double scale, int causal, int mut,
                     double* p, double* oi, int64_t* n_out)
{
    const int64_t n = m_keys(i, sk, causal, mut);
    for (int64_t j = 0; j < n; ++j) {
        const double dp = (mut == FM_K_TRANSPOSED) ? m_dot(qi, kh + j, d, sk)
                                                   : m_dot(qi, kh + j * d, d, 1);
        p[j] = (mut == FM_NO_SCALE) ? dp : scale * dp;
    }
    double m = -INFINITY;
    if (mut == FM_MAX_LAST) {
        m = (n > 0) ? p[n - 1] : -INFINITY;
    } else {
        for (int64_t j = 0; j < n; ++j)
            if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = (mut == FM_EXP_SIGN) ? exp(m - p[j]) : exp(p[j] - m);
        l += p[j];
    }
    for (int64_t x = 0; x < d; ++x) oi[x] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t row = (mut == FM_V_ROW_OFF && j + 1 < sk) ? j + 1 : j;
        for (int64_t x = 0; x < d; ++x) oi[x] += p[j] * vh[row * d + x];
    }
    if (mut != FM_NO_NORMALISE)
        for (int64_t x = 0; x < d; ++x) oi[x] /= l;
    for (int64_t j = 0; j < n; ++j) p[j] /= l;
    if (n_out) *n_out = n;
    return (mut == FM_LSE_NO_MAX) ? log(l) : m + log(l);
}

int oracle_attn_mutant(const double* q, const double* k, const double* v,
                       double* o, double* lse, int64_t b, int64_t h,
                       int64_t sq, int64_t sk, int64_t d, double scale,
                       int causal, int mutant, int nthreads)
{
    (void)nthreads;
    if (!q || !k || !v || !o || !lse || b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || d <= 0)
        return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)sk);
    if (!p) return -1;
    for (int64_t bh = 0; bh < b * h; ++bh)
        for (int64_t i = 0; i < sq; ++i)
            lse[bh * sq + i] = m_row(q + (bh * sq + i) * d, k + bh * sk * d, v + bh * sk * d, i,
                                     sk, d, scale, causal ? 1 : 0, mutant, p,
                                     o + (bh * sq + i) * d, NULL);
    free(p);
    return 0;
}

int oracle_attn_bwd_mutant(const double* q, const double* k, const double* v,
                           const double* dout, double* dq, double* dk, double* dv,
                           int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d,
                           double scale, int causal, int mutant)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || b <= 0 || h <= 0 || sq <= 0 ||
        sk <= 0 || d <= 0)
        return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)sk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)sk);
    double* oi = (double*)malloc(sizeof(double) * (size_t)d);
    if (!p || !dp || !oi) { free(p); free(dp); free(oi); return -1; }
    for (int64_t bh = 0; bh < b * h; ++bh) {
        const double* kh = k + bh * sk * d;
        const double* vh = v + bh * sk * d;
        double* dkh = dk + bh * sk * d;
        double* dvh = dv + bh * sk * d;
        for (int64_t x = 0; x < sk * d; ++x) { dkh[x] = 0.0; dvh[x] = 0.0; }
        for (int64_t i = 0; i < sq; ++i) {
            const double* qi = q + (bh * sq + i) * d;
            const double* gi = dout + (bh * sq + i) * d;
            double* dqi = dq + (bh * sq + i) * d;
            int64_t n = 0;
            (void)m_row(qi, kh, vh, i, sk, d, scale, causal ? 1 : 0, FM_NONE, p, oi, &n);
            double Di = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                dp[j] = m_dot(gi, vh + j * d, d, 1);
                Di += p[j] * dp[j];
            }
            for (int64_t x = 0; x < d; ++x) dqi[x] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double ds = p[j] * (mutant == BM_NO_D ? dp[j] : dp[j] - Di);
                const double* src = (mutant == BM_DQ_USES_V) ? vh + j * d : kh + j * d;
                const double wv = (mutant == BM_DV_USES_DP) ? dp[j] : p[j];
                const double sc_k = (mutant == BM_DK_NO_SCALE) ? 1.0 : scale;
                for (int64_t x = 0; x < d; ++x) {
                    dqi[x] += scale * ds * src[x];
                    dkh[j * d + x] += sc_k * ds * qi[x];
                    dvh[j * d + x] += wv * gi[x];
                }
            }
        }
    }
    free(p); free(dp); free(oi);
    return 0;
}

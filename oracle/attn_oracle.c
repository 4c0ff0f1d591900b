/*
 * attn_oracle.c -- fp64 CPU oracle for exact attention (test infrastructure).
 *
 * THIS FILE IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load it.  The GPU library never
 * links, calls or includes anything from here, and nothing here is shared
 * with the GPU path (no headers, helpers or tables).
 *
 * What it computes (page "flash-attn 实现 prefill 阶段", section 问题分析,
 * the attention formula):
 *
 *     O = softmax(scale * Q K^T) V      per (batch, head) slice of [b,h,s,d]
 *
 * with the softmax taken along the key axis after subtracting the row
 * maximum (page "flash.cu", forward_kernel: the score is the dot product
 * times softmax_scale, then exp(score - row max)).  The row log-sum-exp is
 * reported as LSE_i = m_i + ln(l_i) in natural-log units.
 *
 * Readings taken where the pages are silent:
 *   - causal mask: key j is allowed for query i iff j <= i (top-left
 *     alignment; identical to bottom-right when sq == sk);
 *   - keys j >= sk do not exist (ragged lengths contribute nothing);
 *   - scale is used exactly as passed (the caller passes 1/sqrt(d)).
 *
 * Functions:
 *   oracle_attn          -- the plain definition (naive; explicit scores,
 *                           max-subtracted softmax, weighted sum of V).
 *   oracle_attn_rows     -- the same definition for a list of rows only
 *                           (sampled parity at full problem sizes).
 *   oracle_attn_probs    -- the normalised softmax matrix P (tiny inputs).
 *   oracle_attn_online_kv_outer
 *                        -- the online-softmax recurrence in the order of
 *                           page "flash.cu" forward_kernel: key/value tile
 *                           outer, query tile inner, with per-row running
 *                           max m (init -inf), sum l (init 0) and a
 *                           normalised O (init 0) updated per tile.
 *   oracle_attn_online_q_outer
 *                        -- the same recurrence with the query tile outer
 *                           and an unnormalised accumulator divided by l at
 *                           the end (the order the FA2 traits described on
 *                           page "05 · kernel 工程与四代演化" section 3 use).
 *   oracle_attn_bwd      -- the gradient of the definition: given dO, the
 *                           derivatives dQ, dK, dV of sum(O * dO) (the pages
 *                           name a backward kernel class but print no formula;
 *                           this is the calculus of the forward definition).
 *
 * The deliberately broken copies the pin tests use to show that every pin
 * bites live in attn_mutants.c, apart from the definition above.
 *
 * All arrays are fp64, contiguous, row-major: q,o [b,h,sq,d]; k,v [b,h,sk,d];
 * lse [b,h,sq].  Return value 0 on success, -1 on invalid arguments.
 * The pages print no worked values for the online forms; their pins are the
 * plain definition above, by brute force over small shapes and tile sizes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* The plain definition for one query row.                                   */
/* ------------------------------------------------------------------------ */

/* number of keys row i may attend to: keys 0 .. limit-1 (all sk keys, or
 * with the causal mask the keys j <= i) */
static inline int64_t key_limit(int64_t i, int64_t sk, int causal)
{
    int64_t lim = sk;
    if (causal && i + 1 < lim) lim = i + 1;
    return lim;
}

static double dot(const double* a, const double* b, int64_t d)
{
    /* four partial sums so the compiler can vectorise without reassociating */
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int64_t x = 0;
    for (; x + 4 <= d; x += 4) {
        s0 += a[x] * b[x];
        s1 += a[x + 1] * b[x + 1];
        s2 += a[x + 2] * b[x + 2];
        s3 += a[x + 3] * b[x + 3];
    }
    for (; x < d; ++x) s0 += a[x] * b[x];
    return (s0 + s1) + (s2 + s3);
}

/* One row of the definition.  qi: the query row [d]; kh, vh: the head's K and
 * V [sk, d]; s: scratch [sk]; oi: output row [d]; returns LSE_i.
 * If p_out is non-NULL it receives the normalised probabilities [sk]
 * (zero for keys the row may not attend to). */
static double attend_row(const double* qi, const double* kh, const double* vh,
                         int64_t i, int64_t sk, int64_t d, double scale,
                         int causal, double* s, double* oi, double* p_out)
{
    const int64_t n = key_limit(i, sk, causal);

    /* scores s_j = scale * (q_i . k_j) */
    for (int64_t j = 0; j < n; ++j) s[j] = scale * dot(qi, kh + j * d, d);

    /* row max m */
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];

    /* p_j = exp(s_j - m), l = sum_j p_j */
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }

    /* o = sum_j p_j v_j / l */
    for (int64_t x = 0; x < d; ++x) oi[x] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const double* vj = vh + j * d;
        for (int64_t x = 0; x < d; ++x) oi[x] += s[j] * vj[x];
    }
    for (int64_t x = 0; x < d; ++x) oi[x] /= l;

    if (p_out)
        for (int64_t j = 0; j < sk; ++j) p_out[j] = (j < n) ? s[j] / l : 0.0;

    /* LSE = m + ln l */
    return m + log(l);
}

/* ------------------------------------------------------------------------ */
/* Threading over rows: each thread takes blocks of rows in a strided order. */
/* ------------------------------------------------------------------------ */

typedef struct {
    const double *q, *k, *v;
    double *o, *lse, *p;
    int64_t bh, sq, sk, d;
    double scale;
    int causal;
    const int64_t* rows; /* optional row list (flat index bh_idx*sq + i) */
    int64_t nrows;
    int tid, nthreads;
    int status;
} job_t;

enum { ROW_BLOCK = 8 };

static void* run_rows(void* arg)
{
    job_t* J = (job_t*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)(J->sk > 0 ? J->sk : 1));
    if (!s) { J->status = -1; return NULL; }
    const int64_t total = J->rows ? J->nrows : J->bh * J->sq;
    const int64_t nblk = (total + ROW_BLOCK - 1) / ROW_BLOCK;
    for (int64_t blk = J->tid; blk < nblk; blk += J->nthreads) {
        const int64_t r0 = blk * ROW_BLOCK;
        const int64_t r1 = (r0 + ROW_BLOCK < total) ? r0 + ROW_BLOCK : total;
        for (int64_t r = r0; r < r1; ++r) {
            const int64_t flat = J->rows ? J->rows[r] : r;
            const int64_t bhi = flat / J->sq, i = flat % J->sq;
            const double* qi = J->q + flat * J->d;
            const double* kh = J->k + bhi * J->sk * J->d;
            const double* vh = J->v + bhi * J->sk * J->d;
            /* outputs are indexed by r for row lists, by flat otherwise */
            double* oi = J->o + r * J->d;
            double* pi = J->p ? J->p + r * J->sk : NULL;
            const double l = attend_row(qi, kh, vh, i, J->sk, J->d, J->scale,
                                        J->causal, s, oi, pi);
            J->lse[r] = l;
        }
    }
    free(s);
    return NULL;
}

static int run_threads(job_t proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        jobs[t].status = 0;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_rows, &jobs[t]) != 0) break;
        started = t;
    }
    /* threads that failed to start: run their share here */
    run_rows(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t) run_rows(&jobs[t]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) return -1;
    return 0;
}

static int bad_dims(int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d)
{
    return b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || d <= 0;
}

/* ------------------------------------------------------------------------ */
/* Public entry points                                                       */
/* ------------------------------------------------------------------------ */

int oracle_attn(const double* q, const double* k, const double* v, double* o,
                double* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                int64_t d, double scale, int causal, int nthreads)
{
    if (!q || !k || !v || !o || !lse || bad_dims(b, h, sq, sk, d)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.p = NULL;
    J.bh = b * h; J.sq = sq; J.sk = sk; J.d = d; J.scale = scale;
    J.causal = causal ? 1 : 0;
    return run_threads(J, nthreads);
}

int oracle_attn_rows(const double* q, const double* k, const double* v,
                     const int64_t* rows, int64_t nrows, double* o,
                     double* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                     int64_t d, double scale, int causal, int nthreads)
{
    if (!q || !k || !v || !rows || !o || !lse || nrows < 0 ||
        bad_dims(b, h, sq, sk, d))
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= b * h * sq) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.p = NULL;
    J.bh = b * h; J.sq = sq; J.sk = sk; J.d = d; J.scale = scale;
    J.causal = causal ? 1 : 0;
    J.rows = rows; J.nrows = nrows;
    return run_threads(J, nthreads);
}

int oracle_attn_probs(const double* q, const double* k, const double* v,
                      double* p, double* o, double* lse, int64_t b, int64_t h,
                      int64_t sq, int64_t sk, int64_t d, double scale,
                      int causal)
{
    if (!q || !k || !v || !p || !o || !lse || bad_dims(b, h, sq, sk, d))
        return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.p = p;
    J.bh = b * h; J.sq = sq; J.sk = sk; J.d = d; J.scale = scale;
    J.causal = causal ? 1 : 0;
    return run_threads(J, 1);
}

/* ------------------------------------------------------------------------ */
/* Online-softmax recurrence, key/value tile outer (page "flash.cu",         */
/* forward_kernel).  State per query row: m (init -inf), l (init 0) and a    */
/* normalised O (init 0).  For each key tile the row's tile scores give a    */
/* tile max mt and tile sum lt of exp(s - mt); then                          */
/*   m' = max(m, mt)                                                         */
/*   l' = e^(m - m') l + e^(mt - m') lt                                      */
/*   O' = ( e^(m - m') l O + e^(mt - m') (P~ V) ) / l'                       */
/* A row with no allowed key in a tile skips that tile (its tile max would   */
/* be -inf; the page's code has no mask so never meets this case).           */
/* ------------------------------------------------------------------------ */

int oracle_attn_online_kv_outer(const double* q, const double* k,
                                const double* v, double* o, double* lse,
                                int64_t b, int64_t h, int64_t sq, int64_t sk,
                                int64_t d, double scale, int causal,
                                int64_t br, int64_t bc)
{
    if (!q || !k || !v || !o || !lse || bad_dims(b, h, sq, sk, d) || br <= 0 ||
        bc <= 0)
        return -1;
    double* m = (double*)malloc(sizeof(double) * (size_t)sq);
    double* l = (double*)malloc(sizeof(double) * (size_t)sq);
    double* st = (double*)malloc(sizeof(double) * (size_t)bc);
    double* pv = (double*)malloc(sizeof(double) * (size_t)d);
    if (!m || !l || !st || !pv) { free(m); free(l); free(st); free(pv); return -1; }

    for (int64_t bh = 0; bh < b * h; ++bh) {
        const double* qh = q + bh * sq * d;
        const double* kh = k + bh * sk * d;
        const double* vh = v + bh * sk * d;
        double* oh = o + bh * sq * d;
        for (int64_t i = 0; i < sq; ++i) { m[i] = -INFINITY; l[i] = 0.0; }
        for (int64_t x = 0; x < sq * d; ++x) oh[x] = 0.0;

        for (int64_t j0 = 0; j0 < sk; j0 += bc) {           /* key tile   */
            const int64_t j1 = (j0 + bc < sk) ? j0 + bc : sk;
            for (int64_t i0 = 0; i0 < sq; i0 += br) {       /* query tile */
                const int64_t i1 = (i0 + br < sq) ? i0 + br : sq;
                for (int64_t i = i0; i < i1; ++i) {
                    const int64_t jend = causal ? ((i + 1 < j1) ? i + 1 : j1) : j1;
                    if (jend <= j0) continue;               /* no allowed key */
                    double mt = -INFINITY;
                    for (int64_t j = j0; j < jend; ++j) {
                        st[j - j0] = scale * dot(qh + i * d, kh + j * d, d);
                        if (st[j - j0] > mt) mt = st[j - j0];
                    }
                    double lt = 0.0;
                    for (int64_t j = j0; j < jend; ++j) {
                        st[j - j0] = exp(st[j - j0] - mt);
                        lt += st[j - j0];
                    }
                    const double mn = (m[i] > mt) ? m[i] : mt;
                    const double a_old = exp(m[i] - mn); /* 0 when m = -inf */
                    const double a_new = exp(mt - mn);
                    const double ln = a_old * l[i] + a_new * lt;
                    for (int64_t x = 0; x < d; ++x) pv[x] = 0.0;
                    for (int64_t j = j0; j < jend; ++j)
                        for (int64_t x = 0; x < d; ++x)
                            pv[x] += st[j - j0] * vh[j * d + x];
                    double* oi = oh + i * d;
                    for (int64_t x = 0; x < d; ++x)
                        oi[x] = (a_old * l[i] * oi[x] + a_new * pv[x]) / ln;
                    m[i] = mn;
                    l[i] = ln;
                }
            }
        }
        for (int64_t i = 0; i < sq; ++i) lse[bh * sq + i] = m[i] + log(l[i]);
    }
    free(m); free(l); free(st); free(pv);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Online-softmax recurrence, query tile outer.  Per row: m (init -inf),     */
/* l (init 0), unnormalised accumulator A (init 0).  For each key tile:      */
/*   m' = max(m, max_j s_j);  alpha = e^(m - m');  p_j = e^(s_j - m')        */
/*   l' = alpha l + sum_j p_j;  A' = alpha A + sum_j p_j v_j                 */
/* and at the end O = A / l, LSE = m + ln l.                                 */
/* ------------------------------------------------------------------------ */

int oracle_attn_online_q_outer(const double* q, const double* k,
                               const double* v, double* o, double* lse,
                               int64_t b, int64_t h, int64_t sq, int64_t sk,
                               int64_t d, double scale, int causal,
                               int64_t br, int64_t bc)
{
    if (!q || !k || !v || !o || !lse || bad_dims(b, h, sq, sk, d) || br <= 0 ||
        bc <= 0)
        return -1;
    double* st = (double*)malloc(sizeof(double) * (size_t)bc);
    if (!st) return -1;

    for (int64_t bh = 0; bh < b * h; ++bh) {
        const double* qh = q + bh * sq * d;
        const double* kh = k + bh * sk * d;
        const double* vh = v + bh * sk * d;
        double* oh = o + bh * sq * d;
        for (int64_t i0 = 0; i0 < sq; i0 += br) {           /* query tile */
            const int64_t i1 = (i0 + br < sq) ? i0 + br : sq;
            for (int64_t i = i0; i < i1; ++i) {
                double m = -INFINITY, l = 0.0;
                double* acc = oh + i * d;
                for (int64_t x = 0; x < d; ++x) acc[x] = 0.0;
                for (int64_t j0 = 0; j0 < sk; j0 += bc) {   /* key tile   */
                    const int64_t j1 = (j0 + bc < sk) ? j0 + bc : sk;
                    const int64_t jend = causal ? ((i + 1 < j1) ? i + 1 : j1) : j1;
                    if (jend <= j0) break;  /* later tiles are masked too */
                    double mt = m;
                    for (int64_t j = j0; j < jend; ++j) {
                        st[j - j0] = scale * dot(qh + i * d, kh + j * d, d);
                        if (st[j - j0] > mt) mt = st[j - j0];
                    }
                    const double alpha = exp(m - mt); /* 0 when m = -inf */
                    l *= alpha;
                    for (int64_t x = 0; x < d; ++x) acc[x] *= alpha;
                    for (int64_t j = j0; j < jend; ++j) {
                        const double p = exp(st[j - j0] - mt);
                        l += p;
                        for (int64_t x = 0; x < d; ++x) acc[x] += p * vh[j * d + x];
                    }
                    m = mt;
                }
                for (int64_t x = 0; x < d; ++x) acc[x] /= l;
                lse[bh * sq + i] = m + log(l);
            }
        }
    }
    free(st);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward: derivatives of L = sum_ij O_ij dO_ij with respect to Q, K, V.   */
/* With P_ij the softmax probabilities of row i (0 for keys it may not see):  */
/*   dV_j  = sum_i P_ij dO_i                                                 */
/*   dP_ij = dO_i . v_j                                                      */
/*   D_i   = sum_j P_ij dP_ij            (equals dO_i . O_i)                 */
/*   dS_ij = P_ij (dP_ij - D_i)          (derivative through the softmax)   */
/*   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i           */
/* Heads run in parallel; each thread owns whole heads.                      */
/* ------------------------------------------------------------------------ */

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    int64_t bh, sq, sk, d;
    double scale;
    int causal, tid, nthreads, status;
} bjob_t;

static void* run_bwd(void* arg)
{
    bjob_t* J = (bjob_t*)arg;
    const int64_t sq = J->sq, sk = J->sk, d = J->d;
    double* s = (double*)malloc(sizeof(double) * (size_t)sk);
    double* p = (double*)malloc(sizeof(double) * (size_t)sk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)sk);
    double* oi = (double*)malloc(sizeof(double) * (size_t)d);
    if (!s || !p || !dp || !oi) {
        J->status = -1;
        free(s); free(p); free(dp); free(oi);
        return NULL;
    }
    for (int64_t hh = J->tid; hh < J->bh; hh += J->nthreads) {
        const double* qh = J->q + hh * sq * d;
        const double* kh = J->k + hh * sk * d;
        const double* vh = J->v + hh * sk * d;
        const double* gh = J->dout + hh * sq * d;
        double* dqh = J->dq + hh * sq * d;
        double* dkh = J->dk + hh * sk * d;
        double* dvh = J->dv + hh * sk * d;
        for (int64_t x = 0; x < sk * d; ++x) { dkh[x] = 0.0; dvh[x] = 0.0; }
        for (int64_t i = 0; i < sq; ++i) {
            const double* qi = qh + i * d;
            const double* gi = gh + i * d;
            (void)attend_row(qi, kh, vh, i, sk, d, J->scale, J->causal, s, oi, p);
            const int64_t n = key_limit(i, sk, J->causal);
            double Di = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                dp[j] = dot(gi, vh + j * d, d);
                Di += p[j] * dp[j];
            }
            double* dqi = dqh + i * d;
            for (int64_t x = 0; x < d; ++x) dqi[x] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double ds = p[j] * (dp[j] - Di);
                const double* kj = kh + j * d;
                double* dkj = dkh + j * d;
                double* dvj = dvh + j * d;
                for (int64_t x = 0; x < d; ++x) {
                    dqi[x] += J->scale * ds * kj[x];
                    dkj[x] += J->scale * ds * qi[x];
                    dvj[x] += p[j] * gi[x];
                }
            }
        }
    }
    free(s); free(p); free(dp); free(oi);
    return NULL;
}

int oracle_attn_bwd(const double* q, const double* k, const double* v,
                    const double* dout, double* dq, double* dk, double* dv,
                    int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d,
                    double scale, int causal, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || bad_dims(b, h, sq, sk, d))
        return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    bjob_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        bjob_t J;
        memset(&J, 0, sizeof J);
        J.q = q; J.k = k; J.v = v; J.dout = dout; J.dq = dq; J.dk = dk; J.dv = dv;
        J.bh = b * h; J.sq = sq; J.sk = sk; J.d = d; J.scale = scale;
        J.causal = causal ? 1 : 0; J.tid = t; J.nthreads = nthreads;
        jobs[t] = J;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_bwd, &jobs[t]) != 0) break;
        started = t;
    }
    run_bwd(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t) run_bwd(&jobs[t]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) return -1;
    return 0;
}

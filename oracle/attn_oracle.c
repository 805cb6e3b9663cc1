/*
 * attn_oracle.c -- fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or table with the GPU library.
 *
 * What it computes is the plain definition of standard (materialising)
 * attention.  The pages present the tiled method as reproducing that result
 * exactly, with no approximation and no loss of accuracy, so the definition
 * itself is the reference:
 *
 *   S = scale * Q K^T      one full score row at a time.  Source: the
 *                          shakilmahmud.com page "Large language models part
 *                          06: FlashAttention -- GPU SRAM, tiling, online
 *                          softmax", section 1 (S is formed, then P, then O).
 *   P = softmax(S)         row-wise, the row maximum m subtracted before
 *                          exponentiating.  Source: unite.ai page "Flash
 *                          Attention: revolutionising transformer
 *                          efficiency", section on the maths behind Flash
 *                          Attention (softmax decomposition).
 *   O = P V                same section 1; the standard-attention recap on the
 *                          unite.ai page.
 *   lse = m + ln(sum_j exp(S_ij - m))
 *                          the pages define no log-sum-exp output; this is the
 *                          natural-log reading, with the scale included.
 *
 * Causal masking is not on the pages either; the reading used here is the
 * autoregressive one with rows and columns aligned at the top-left corner:
 * query i sees key j iff j <= i.  A row whose keys are all masked (only
 * possible when Nk == 0, which the entry points reject) would give O = 0,
 * lse = -inf.
 *
 * Everything is evaluated in IEEE double precision, row by row, over the
 * whole key range; there is no tiling, no online rescaling and no reordering
 * beyond the definition.  Threads (POSIX) split the independent rows.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One query row: fills p[0..nk) with the probability row, returns m and l. */
static void probs_row(const double *qi, const double *k, int64_t nk,
                      int64_t d, double scale, int causal, int64_t i,
                      double *p, double *m_out, double *l_out)
{
    /* scores: s_j = scale * <q_i, k_j>, masked keys at -inf */
    for (int64_t j = 0; j < nk; ++j) {
        if (causal && j > i) {
            p[j] = -INFINITY;
            continue;
        }
        const double *kj = k + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * kj[c];
        p[j] = scale * dot;
    }
    /* safe softmax: subtract the row maximum before exponentiating */
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j)
        if (p[j] > m)
            m = p[j];
    if (m == -INFINITY) { /* every key masked */
        for (int64_t j = 0; j < nk; ++j)
            p[j] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        p[j] = exp(p[j] - m); /* exp(-inf) == 0 for masked keys */
        l += p[j];
    }
    for (int64_t j = 0; j < nk; ++j)
        p[j] /= l;
    *m_out = m;
    *l_out = l;
}

/* O row = P row times V; lse = m + ln l. */
static void attend_row(const double *qi, const double *k, const double *v,
                       int64_t nk, int64_t d, double scale, int causal,
                       int64_t i, double *p, double *oi, double *lse_i)
{
    double m, l;
    probs_row(qi, k, nk, d, scale, causal, i, p, &m, &l);
    for (int64_t c = 0; c < d; ++c)
        oi[c] = 0.0;
    /* masked keys have p == 0 by definition, so the sum runs over the
       visible keys only */
    int64_t jend = (causal && i + 1 < nk) ? i + 1 : nk;
    for (int64_t j = 0; j < jend; ++j) {
        const double *vj = v + j * d;
        for (int64_t c = 0; c < d; ++c)
            oi[c] += p[j] * vj[c];
    }
    if (lse_i)
        *lse_i = (l > 0.0) ? m + log(l) : -INFINITY;
}

int oracle_default_threads(void)
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0)
            return n;
    }
    return 1;
}

/* ---- work splitting over rows -------------------------------------- */

typedef struct {
    /* full-tensor mode */
    const double *q, *k, *v;
    double *o, *lse;
    int64_t nq, nk, d;
    double scale;
    int causal;
    /* row list mode (rows != NULL): q holds nrows gathered rows */
    const int64_t *rows;
    /* rows are claimed in chunks from this counter */
    int64_t total;
    int64_t next;
    pthread_mutex_t lock;
    int failed;
} job_t;

static int64_t claim(job_t *jb, int64_t chunk, int64_t *end)
{
    pthread_mutex_lock(&jb->lock);
    int64_t s = jb->next;
    jb->next = s + chunk < jb->total ? s + chunk : jb->total;
    *end = jb->next;
    pthread_mutex_unlock(&jb->lock);
    return s;
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)(jb->nk > 0 ? jb->nk : 1));
    if (!p) {
        pthread_mutex_lock(&jb->lock);
        jb->failed = 1;
        pthread_mutex_unlock(&jb->lock);
        return NULL;
    }
    for (;;) {
        int64_t end;
        int64_t s = claim(jb, 16, &end);
        if (s >= end)
            break;
        for (int64_t r = s; r < end; ++r) {
            if (jb->rows) {
                /* row list: one head's K/V, gathered query rows */
                attend_row(jb->q + r * jb->d, jb->k, jb->v, jb->nk, jb->d,
                           jb->scale, jb->causal, jb->rows[r], p,
                           jb->o + r * jb->d, jb->lse ? jb->lse + r : NULL);
            } else {
                /* full tensor: r enumerates (head, query row) */
                int64_t head = r / jb->nq, i = r % jb->nq;
                const double *kh = jb->k + head * jb->nk * jb->d;
                const double *vh = jb->v + head * jb->nk * jb->d;
                attend_row(jb->q + r * jb->d, kh, vh, jb->nk, jb->d,
                           jb->scale, jb->causal, i, p, jb->o + r * jb->d,
                           jb->lse ? jb->lse + r : NULL);
            }
        }
    }
    free(p);
    return NULL;
}

static int run(job_t *jb, int nthreads)
{
    if (nthreads <= 0)
        nthreads = oracle_default_threads();
    if (nthreads > jb->total && jb->total > 0)
        nthreads = (int)jb->total;
    if (nthreads < 1)
        nthreads = 1;
    pthread_mutex_init(&jb->lock, NULL);
    jb->next = 0;
    jb->failed = 0;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!th)
        return -1;
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, worker, jb) == 0)
            ++started;
    worker(jb); /* the calling thread works too */
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&jb->lock);
    return jb->failed ? -1 : started + 1;
}

/*
 * Full attention over nh independent heads.
 *   q: [nh][nq][d], k, v: [nh][nk][d], o: [nh][nq][d], lse: [nh][nq] or NULL.
 * Returns the number of threads used, or -1 on allocation failure / bad size.
 */
int oracle_attention_f64(const double *q, const double *k, const double *v,
                         double *o, double *lse, int64_t nh, int64_t nq,
                         int64_t nk, int64_t d, double scale, int causal,
                         int nthreads)
{
    if (nh < 0 || nq < 0 || nk < 1 || d < 1)
        return -1;
    job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v; jb.o = o; jb.lse = lse;
    jb.nq = nq; jb.nk = nk; jb.d = d; jb.scale = scale; jb.causal = causal;
    jb.rows = NULL;
    jb.total = nh * nq;
    return run(&jb, nthreads);
}

/*
 * Selected query rows of one head.
 *   q_rows: [nrows][d] (the query vectors), rows: [nrows] their row indices
 *   (used only by the causal mask), k, v: [nk][d], o: [nrows][d],
 *   lse: [nrows] or NULL.
 */
int oracle_attention_rows_f64(const double *q_rows, const int64_t *rows,
                              int64_t nrows, const double *k, const double *v,
                              int64_t nk, int64_t d, double scale, int causal,
                              double *o, double *lse, int nthreads)
{
    if (nrows < 0 || nk < 1 || d < 1 || !rows)
        return -1;
    job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q_rows; jb.k = k; jb.v = v; jb.o = o; jb.lse = lse;
    jb.nq = nrows; jb.nk = nk; jb.d = d; jb.scale = scale; jb.causal = causal;
    jb.rows = rows;
    jb.total = nrows;
    return run(&jb, nthreads);
}

/*
 * The probability matrix P of one head (small sizes only: nq * nk doubles).
 *   q: [nq][d], k: [nk][d], p: [nq][nk], m, l: [nq] (row max and the
 *   sum of exp(s - m)), either may be NULL.
 */
int oracle_probs_f64(const double *q, const double *k, int64_t nq, int64_t nk,
                     int64_t d, double scale, int causal, double *p,
                     double *m, double *l)
{
    if (nq < 0 || nk < 1 || d < 1)
        return -1;
    for (int64_t i = 0; i < nq; ++i) {
        double mi, li;
        probs_row(q + i * d, k, nk, d, scale, causal, i, p + i * nk, &mi, &li);
        if (m)
            m[i] = mi;
        if (l)
            l[i] = li;
    }
    return 0;
}

/* ==== gradients ======================================================
 *
 * The pages say that the method recomputes parts of the attention matrix in
 * the backward pass instead of storing it (unite.ai page, section "Enter
 * Flash Attention", the recomputation idea) and that FlashAttention-2 made
 * that backward pass nearly as fast as the forward one (same page,
 * "FlashAttention-2", second improvement).  They give no formula for it, so
 * the reference is the plain definition: the exact gradient of the forward
 * definition above with respect to Q, K and V, for an incoming gradient dO
 * of O (the derivative of a loss L with dL/dO = dO).  Written out per head,
 * with P the probability matrix of the forward pass:
 *
 *   dV_j  = sum_i P_ij dO_i                       (O_i = sum_j P_ij V_j)
 *   dP_ij = dO_i . V_j
 *   dS_ij = P_ij (dP_ij - D_i),  D_i = sum_j P_ij dP_ij
 *                                  (Jacobian of the row softmax)
 *   dQ_i  = scale * sum_j dS_ij K_j                (S_ij = scale Q_i . K_j)
 *   dK_j  = scale * sum_i dS_ij Q_i
 *
 * Masked entries have P_ij = 0 and so contribute nothing.  Everything is in
 * double precision, one query row at a time over all of its keys.  Rows are
 * split statically over the threads; each thread sums its rows' dK and dV
 * contributions privately and the partial sums are added in thread order,
 * so a given thread count always gives the same bits.
 */

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *delta;
    double *dk_part, *dv_part; /* this thread's [nk][d] partial sums */
    int64_t r0, r1, nk, d;
    double scale;
    int causal;
    int failed;
} bwd_job_t;

static void *bwd_worker(void *arg)
{
    bwd_job_t *jb = (bwd_job_t *)arg;
    const int64_t nk = jb->nk, d = jb->d;
    double *p = (double *)malloc(sizeof(double) * (size_t)nk);
    double *dp = (double *)malloc(sizeof(double) * (size_t)nk);
    if (!p || !dp) {
        free(p);
        free(dp);
        jb->failed = 1;
        return NULL;
    }
    memset(jb->dk_part, 0, sizeof(double) * (size_t)(nk * d));
    memset(jb->dv_part, 0, sizeof(double) * (size_t)(nk * d));
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const double *qi = jb->q + i * d;
        const double *gi = jb->dout + i * d;
        double m, l;
        probs_row(qi, jb->k, nk, d, jb->scale, jb->causal, i, p, &m, &l);
        /* dP_ij and D_i */
        double di = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            const double *vj = jb->v + j * d;
            double s = 0.0;
            for (int64_t c = 0; c < d; ++c)
                s += gi[c] * vj[c];
            dp[j] = s;
            di += p[j] * s;
        }
        if (jb->delta)
            jb->delta[i] = di;
        double *dqi = jb->dq + i * d;
        for (int64_t c = 0; c < d; ++c)
            dqi[c] = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            const double ds = p[j] * (dp[j] - di);
            const double *kj = jb->k + j * d;
            double *dkj = jb->dk_part + j * d;
            double *dvj = jb->dv_part + j * d;
            for (int64_t c = 0; c < d; ++c) {
                dqi[c] += ds * kj[c];
                dkj[c] += ds * qi[c];
                dvj[c] += p[j] * gi[c];
            }
        }
        for (int64_t c = 0; c < d; ++c)
            dqi[c] *= jb->scale;
    }
    free(p);
    free(dp);
    return NULL;
}

/*
 * Gradients of every head.
 *   q, dout, dq: [nh][nq][d];  k, v, dk, dv: [nh][nk][d];
 *   delta: [nh][nq] (D_i above) or NULL.
 * Returns the number of threads used, or -1 on allocation failure / bad size.
 */
int oracle_attention_bwd_f64(const double *q, const double *k, const double *v,
                             const double *dout, double *dq, double *dk,
                             double *dv, double *delta, int64_t nh, int64_t nq,
                             int64_t nk, int64_t d, double scale, int causal,
                             int nthreads)
{
    if (nh < 0 || nq < 1 || nk < 1 || d < 1)
        return -1;
    if (nthreads <= 0)
        nthreads = oracle_default_threads();
    if (nthreads > nq)
        nthreads = (int)nq;
    const size_t part = (size_t)(nk * d);
    double *parts = (double *)malloc(sizeof(double) * part * 2 * (size_t)nthreads);
    bwd_job_t *jobs = (bwd_job_t *)calloc((size_t)nthreads, sizeof(bwd_job_t));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int *started = (int *)calloc((size_t)nthreads, sizeof(int));
    int rc = nthreads;
    if (!parts || !jobs || !th || !started) {
        rc = -1;
        goto out;
    }
    for (int64_t h = 0; h < nh && rc > 0; ++h) {
        for (int t = 0; t < nthreads; ++t) {
            bwd_job_t *jb = &jobs[t];
            jb->q = q + h * nq * d;
            jb->dout = dout + h * nq * d;
            jb->k = k + h * nk * d;
            jb->v = v + h * nk * d;
            jb->dq = dq + h * nq * d;
            jb->delta = delta ? delta + h * nq : NULL;
            jb->dk_part = parts + (size_t)(2 * t) * part;
            jb->dv_part = parts + (size_t)(2 * t + 1) * part;
            jb->r0 = nq * t / nthreads;
            jb->r1 = nq * (t + 1) / nthreads;
            jb->nk = nk;
            jb->d = d;
            jb->scale = scale;
            jb->causal = causal;
            jb->failed = 0;
            started[t] = 0;
        }
        for (int t = 1; t < nthreads; ++t)
            started[t] = pthread_create(&th[t], NULL, bwd_worker, &jobs[t]) == 0;
        bwd_worker(&jobs[0]);
        for (int t = 1; t < nthreads; ++t) {
            if (started[t])
                pthread_join(th[t], NULL);
            else
                bwd_worker(&jobs[t]); /* could not start: run it here */
        }
        double *dkh = dk + h * nk * d, *dvh = dv + h * nk * d;
        for (size_t e = 0; e < part; ++e) {
            double sk = 0.0, sv = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                sk += parts[(size_t)(2 * t) * part + e];
                sv += parts[(size_t)(2 * t + 1) * part + e];
            }
            dkh[e] = scale * sk;
            dvh[e] = sv;
        }
        for (int t = 0; t < nthreads; ++t)
            if (jobs[t].failed)
                rc = -1;
    }
out:
    free(parts);
    free(jobs);
    free(th);
    free(started);
    return rc;
}

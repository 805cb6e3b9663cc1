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
 * Masked entries have P_ij = 0 and so contribute nothing: the sums below
 * run over the visible pairs only (adding an exact zero changes no sum).
 * Everything is in double precision.  Two passes, each over independent
 * items split between threads:
 *   rows:  for each query row i, P_i (with its m_i and l_i), dP_i, D_i and
 *          dQ_i, every sum over the keys j in increasing order;
 *   keys:  for each key j, dK_j and dV_j summed over the query rows i in
 *          increasing order, with P_ij recomputed from the same operations
 *          as in the row pass (the same bits) and D_i from that pass.
 * No sum is split between threads, so the result does not depend on the
 * thread count.
 */

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv, *delta;
    double *m, *l;          /* [nh][nq] row statistics from the row pass */
    int64_t nq, nk, d;
    double scale;
    int causal;
    int keys;               /* 0: row pass, 1: key pass */
    int64_t total, next;
    pthread_mutex_t lock;
    int failed;
} bwd_job_t;

static int64_t bwd_claim(bwd_job_t *jb, int64_t chunk, int64_t *end)
{
    pthread_mutex_lock(&jb->lock);
    int64_t s = jb->next;
    jb->next = s + chunk < jb->total ? s + chunk : jb->total;
    *end = jb->next;
    pthread_mutex_unlock(&jb->lock);
    return s;
}

/* Row pass for query row i of one head: P_i, D_i, dQ_i, and m_i, l_i. */
static void bwd_row(const bwd_job_t *jb, int64_t head, int64_t i, double *p,
                    double *dp)
{
    const int64_t nq = jb->nq, nk = jb->nk, d = jb->d;
    const double *qi = jb->q + (head * nq + i) * d;
    const double *gi = jb->dout + (head * nq + i) * d;
    const double *kh = jb->k + head * nk * d;
    const double *vh = jb->v + head * nk * d;
    double m, l;
    probs_row(qi, kh, nk, d, jb->scale, jb->causal, i, p, &m, &l);
    const int64_t jend = (jb->causal && i + 1 < nk) ? i + 1 : nk;
    /* dP_ij = dO_i . V_j and D_i = sum_j P_ij dP_ij */
    double di = 0.0;
    for (int64_t j = 0; j < jend; ++j) {
        const double *vj = vh + j * d;
        double s = 0.0;
        for (int64_t c = 0; c < d; ++c)
            s += gi[c] * vj[c];
        dp[j] = s;
        di += p[j] * s;
    }
    /* dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j */
    double *dqi = jb->dq + (head * nq + i) * d;
    for (int64_t c = 0; c < d; ++c)
        dqi[c] = 0.0;
    for (int64_t j = 0; j < jend; ++j) {
        const double ds = p[j] * (dp[j] - di);
        const double *kj = kh + j * d;
        for (int64_t c = 0; c < d; ++c)
            dqi[c] += ds * kj[c];
    }
    for (int64_t c = 0; c < d; ++c)
        dqi[c] *= jb->scale;
    jb->delta[head * nq + i] = di;
    jb->m[head * nq + i] = m;
    jb->l[head * nq + i] = l;
}

/* Key pass for key j of one head: dK_j and dV_j. */
static void bwd_key(const bwd_job_t *jb, int64_t head, int64_t j)
{
    const int64_t nq = jb->nq, nk = jb->nk, d = jb->d;
    const double *kj = jb->k + (head * nk + j) * d;
    const double *vj = jb->v + (head * nk + j) * d;
    double *dkj = jb->dk + (head * nk + j) * d;
    double *dvj = jb->dv + (head * nk + j) * d;
    for (int64_t c = 0; c < d; ++c) {
        dkj[c] = 0.0;
        dvj[c] = 0.0;
    }
    /* causal: key j is visible from the rows i >= j */
    for (int64_t i = jb->causal ? j : 0; i < nq; ++i) {
        const double li = jb->l[head * nq + i];
        if (!(li > 0.0))
            continue; /* a row with no visible key has P = 0 */
        const double *qi = jb->q + (head * nq + i) * d;
        const double *gi = jb->dout + (head * nq + i) * d;
        /* P_ij exactly as the row pass formed it */
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * kj[c];
        double pij = jb->scale * dot;
        pij = exp(pij - jb->m[head * nq + i]);
        pij /= li;
        double dpij = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dpij += gi[c] * vj[c];
        const double ds = pij * (dpij - jb->delta[head * nq + i]);
        for (int64_t c = 0; c < d; ++c) {
            dkj[c] += ds * qi[c];
            dvj[c] += pij * gi[c];
        }
    }
    for (int64_t c = 0; c < d; ++c)
        dkj[c] *= jb->scale;
}

static void *bwd_worker(void *arg)
{
    bwd_job_t *jb = (bwd_job_t *)arg;
    const int64_t nk = jb->nk;
    double *p = NULL, *dp = NULL;
    if (!jb->keys) {
        p = (double *)malloc(sizeof(double) * (size_t)nk);
        dp = (double *)malloc(sizeof(double) * (size_t)nk);
        if (!p || !dp) {
            free(p);
            free(dp);
            pthread_mutex_lock(&jb->lock);
            jb->failed = 1;
            pthread_mutex_unlock(&jb->lock);
            return NULL;
        }
    }
    for (;;) {
        int64_t end;
        int64_t s = bwd_claim(jb, 16, &end);
        if (s >= end)
            break;
        for (int64_t r = s; r < end; ++r) {
            if (jb->keys)
                bwd_key(jb, r / nk, r % nk);
            else
                bwd_row(jb, r / jb->nq, r % jb->nq, p, dp);
        }
    }
    free(p);
    free(dp);
    return NULL;
}

static int bwd_run(bwd_job_t *jb, int nthreads)
{
    if (nthreads > jb->total && jb->total > 0)
        nthreads = (int)jb->total;
    if (nthreads < 1)
        nthreads = 1;
    pthread_mutex_init(&jb->lock, NULL);
    jb->next = 0;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!th) {
        pthread_mutex_destroy(&jb->lock);
        return -1;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[started], NULL, bwd_worker, jb) == 0)
            ++started;
    bwd_worker(jb); /* the calling thread works too */
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&jb->lock);
    return jb->failed ? -1 : started + 1;
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
    const size_t rows = (size_t)(nh * nq);
    double *stats = (double *)malloc(sizeof(double) * (rows ? rows : 1) * 3);
    if (!stats)
        return -1;
    bwd_job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.q = q; jb.k = k; jb.v = v; jb.dout = dout;
    jb.dq = dq; jb.dk = dk; jb.dv = dv;
    jb.delta = stats;
    jb.m = stats + rows;
    jb.l = stats + 2 * rows;
    jb.nq = nq; jb.nk = nk; jb.d = d;
    jb.scale = scale;
    jb.causal = causal;
    jb.keys = 0;
    jb.total = nh * nq;
    int rc = bwd_run(&jb, nthreads);
    if (rc > 0) {
        jb.keys = 1;
        jb.total = nh * nk;
        jb.failed = 0;
        int rc2 = bwd_run(&jb, nthreads);
        rc = rc2 < 0 ? -1 : (rc2 > rc ? rc2 : rc);
    }
    if (rc > 0 && delta)
        memcpy(delta, stats, sizeof(double) * rows);
    free(stats);
    return rc;
}

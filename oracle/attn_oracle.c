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

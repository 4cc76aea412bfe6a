/*
 * swa_oracle.c -- plain fp64 CPU oracle for SWA(w,s) causal softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the GPU library, and nothing in the GPU library loads it.
 *
 * What it computes (all positions 0-based):
 *
 *   SWA(w,s): query t attends to the most recent w tokens and to the first s tokens
 *   ("sinks").  Source: page "滑动窗口注意力（SWA）配 sinks 比 post-training 线性注意力
 *   更划算" (papers.ananclaw.com explainer of arXiv 2608.28444), section 核心方法 1,
 *   the notation paragraph, the x_t equation and the swa_mask pseudocode.
 *
 *   The window length counts the query itself: token t sees t-W+1 .. t.  Source: page
 *   "从长文档摘要说起" (wiblog.cn, sliding-window-attention-long-context-inference),
 *   section "SWA 的核心机制：局部窗口与跨层感受野".
 *
 *   Readings taken where the pages are open (each listed in the design doc):
 *     - the allowed set is intersected with causality (i <= t), so a query before
 *       position s never sees a later sink;
 *     - sinks and window form a union: a key in both is counted once;
 *     - the softmax is normalised over the allowed set only, with no extra logit;
 *     - conv = ADDITIVE: w_loc = w (w recent keys plus s sinks, as in the "64+4=68
 *       tokens" of the first page's deployment notes);
 *       conv = TOTAL: w_loc = w - s (a total window of w that includes the s sinks,
 *       as the PaperWeekly page "几亿Token白练了？" phrases SWA(64,4));
 *     - grouped-query attention maps q-head h to kv-head floor(h / (Hq/Hkv)).
 *
 * Algorithm per output row (b, t, h): enumerate i = 0..t, keep i when allowed(t, i),
 * form the logit scale * <q_t, k_i>, subtract the row maximum, exponentiate, divide by
 * the sum, and weight v_i.  This is the two-pass max/sum softmax written out; no tiling,
 * no online rescaling, no reordering of the sums beyond increasing i.
 *
 * Parity pins live in tests/test_oracle_pins.py; every function here is pinned there.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CONV_ADDITIVE 0
#define ORACLE_CONV_TOTAL 1

/* Local window length from (w, s, convention).  Returns 0 on success, -1 if the
 * combination leaves no local window (w_loc < 1) or an argument is out of range. */
int swa_oracle_local_window(int64_t w, int64_t s, int conv, int64_t *w_loc)
{
    int64_t wl;
    if (w < 1 || s < 0 || w_loc == NULL)
        return -1;
    if (conv == ORACLE_CONV_ADDITIVE)
        wl = w;
    else if (conv == ORACLE_CONV_TOTAL)
        wl = w - s;
    else
        return -1;
    if (wl < 1)
        return -1;
    *w_loc = wl;
    return 0;
}

/* The allowed-key predicate A(t): causal, and either inside the local window of the
 * w_loc most recent keys (self included) or one of the first s keys. */
int swa_oracle_allowed(int64_t t, int64_t i, int64_t w_loc, int64_t s)
{
    if (i < 0 || i > t)
        return 0;
    if (i >= t - w_loc + 1)
        return 1;
    if (i < s)
        return 1;
    return 0;
}

/* Dense L x L 0/1 matrix of the predicate, row t = query, column i = key. */
void swa_oracle_mask(uint8_t *mask, int64_t L, int64_t w_loc, int64_t s)
{
    for (int64_t t = 0; t < L; ++t)
        for (int64_t i = 0; i < L; ++i)
            mask[t * L + i] = (uint8_t)swa_oracle_allowed(t, i, w_loc, s);
}

/* Softmax weights of one query row over keys 0..t.
 *   q: d values; k: key rows, row i starts at k + i * k_stride; p: t+1 outputs.
 * p[i] = 0 for keys outside A(t).  Returns |A(t)|. */
int64_t swa_oracle_row_weights(const double *q, const double *k, int64_t k_stride, int d,
                               int64_t t, int64_t w_loc, int64_t s, double scale, double *p)
{
    double m = -INFINITY, den = 0.0;
    int64_t n = 0;
    for (int64_t i = 0; i <= t; ++i) {
        p[i] = 0.0;
        if (!swa_oracle_allowed(t, i, w_loc, s))
            continue;
        const double *ki = k + i * k_stride;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += q[c] * ki[c];
        p[i] = scale * dot; /* logit, overwritten by the weight below */
        if (p[i] > m)
            m = p[i];
        ++n;
    }
    for (int64_t i = 0; i <= t; ++i) {
        if (!swa_oracle_allowed(t, i, w_loc, s))
            continue;
        p[i] = exp(p[i] - m);
        den += p[i];
    }
    for (int64_t i = 0; i <= t; ++i)
        if (swa_oracle_allowed(t, i, w_loc, s))
            p[i] /= den;
    return n;
}

/* x = sum_i p[i] v_i over the allowed keys; v row i starts at v + i * v_stride. */
static void weighted_sum(const double *p, const double *v, int64_t v_stride, int d, int64_t t,
                         int64_t w_loc, int64_t s, double *x)
{
    for (int c = 0; c < d; ++c)
        x[c] = 0.0;
    for (int64_t i = 0; i <= t; ++i) {
        if (!swa_oracle_allowed(t, i, w_loc, s))
            continue;
        const double *vi = v + i * v_stride;
        for (int c = 0; c < d; ++c)
            x[c] += p[i] * vi[c];
    }
}

typedef struct {
    const double *q, *k, *v;
    double *out;
    int64_t B, Hq, Hkv, L, d, w_loc, s;
    int64_t t_lo, t_hi; /* rows computed: t_lo <= t < t_hi (out holds those rows only) */
    double scale;
    int64_t nthreads, tid;
    int status;
} prefill_job;

static void *prefill_worker(void *arg)
{
    prefill_job *j = (prefill_job *)arg;
    const int64_t group = j->Hq / j->Hkv;
    const int64_t nt = j->t_hi - j->t_lo;
    const int64_t rows = j->B * nt * j->Hq;
    const int64_t block = 16;
    double *p = (double *)malloc((size_t)j->L * sizeof(double));
    if (p == NULL) {
        j->status = -2;
        return NULL;
    }
    /* Static interleaving of 16-row blocks over threads; rows are independent. */
    for (int64_t r0 = j->tid * block; r0 < rows; r0 += j->nthreads * block) {
        for (int64_t r = r0; r < r0 + block && r < rows; ++r) {
            const int64_t h = r % j->Hq;
            const int64_t t = j->t_lo + (r / j->Hq) % nt;
            const int64_t b = r / (j->Hq * nt);
            const int64_t kvh = h / group;
            const double *qr = j->q + ((b * j->L + t) * j->Hq + h) * j->d;
            const double *kb = j->k + (b * j->L * j->Hkv + kvh) * j->d;
            const double *vb = j->v + (b * j->L * j->Hkv + kvh) * j->d;
            const int64_t kv_stride = j->Hkv * j->d;
            double *xr = j->out + ((b * nt + (t - j->t_lo)) * j->Hq + h) * j->d;
            swa_oracle_row_weights(qr, kb, kv_stride, (int)j->d, t, j->w_loc, j->s, j->scale, p);
            weighted_sum(p, vb, kv_stride, (int)j->d, t, j->w_loc, j->s, xr);
        }
    }
    free(p);
    j->status = 0;
    return NULL;
}

/* SWA(w,s) attention rows t_lo <= t < t_hi of whole sequences (every batch item and q-head).
 *   q:   [B][L][Hq][d]  k, v: [B][L][Hkv][d]  out: [B][t_hi - t_lo][Hq][d], all fp64, row-major.
 * Each row is computed exactly as in swa_oracle_prefill (rows are independent).
 * Returns 0, or -1 on bad arguments, -2 if a thread could not be started. */
int swa_oracle_prefill_rows(const double *q, const double *k, const double *v, double *out,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t w_loc,
                            int64_t s, double scale, int64_t t_lo, int64_t t_hi, int nthreads)
{
    if (!q || !k || !v || !out || B < 1 || L < 1 || d < 1 || Hkv < 1 || Hq < Hkv ||
        Hq % Hkv != 0 || w_loc < 1 || s < 0 || t_lo < 0 || t_hi > L || t_lo >= t_hi)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    prefill_job *jobs = (prefill_job *)calloc((size_t)nthreads, sizeof(prefill_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -2;
    }
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        prefill_job j = {q, k, v, out, B, Hq, Hkv, L, d, w_loc, s, t_lo, t_hi, scale, nthreads, i, -3};
        jobs[i] = j;
        if (pthread_create(&th[i], NULL, prefill_worker, &jobs[i]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(th[i], NULL);
        if (jobs[i].status != 0)
            rc = -2;
    }
    if (started < nthreads)
        rc = -2;
    free(jobs);
    free(th);
    return rc;
}

/* Whole-sequence SWA(w,s) attention: every row t < L.
 *   q:   [B][L][Hq][d]  k, v: [B][L][Hkv][d]  out: [B][L][Hq][d], all fp64, row-major.
 * Returns 0, or -1 on bad arguments, -2 if a thread could not be started. */
int swa_oracle_prefill(const double *q, const double *k, const double *v, double *out, int64_t B,
                       int64_t Hq, int64_t Hkv, int64_t L, int64_t d, int64_t w_loc, int64_t s,
                       double scale, int nthreads)
{
    return swa_oracle_prefill_rows(q, k, v, out, B, Hq, Hkv, L, d, w_loc, s, scale, 0, L, nthreads);
}

/* Log of the softmax denominator of rows t_lo <= t < t_hi: for every (b, t, h),
 *   lse[b][t - t_lo][h] = ln sum_{i in A(t)} exp(scale * <q[b][t][h], k[b][i][g(h)]>),
 * taken as m + ln sum exp(l_i - m) with m the row maximum of the logits l_i (fp64).
 *   q: [B][L][Hq][d]  k: [B][L][Hkv][d]  lse: [B][t_hi - t_lo][Hq].
 * Returns 0, or -1 on bad arguments. */
int swa_oracle_lse_rows(const double *q, const double *k, double *lse, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t L, int64_t d, int64_t w_loc, int64_t s, double scale,
                        int64_t t_lo, int64_t t_hi)
{
    if (!q || !k || !lse || B < 1 || L < 1 || d < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 ||
        w_loc < 1 || s < 0 || t_lo < 0 || t_hi > L || t_lo >= t_hi)
        return -1;
    const int64_t group = Hq / Hkv;
    double *lg = (double *)malloc((size_t)L * sizeof(double));
    if (!lg)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = t_lo; t < t_hi; ++t)
            for (int64_t h = 0; h < Hq; ++h) {
                const double *qr = q + ((b * L + t) * Hq + h) * d;
                double m = -INFINITY, sum = 0.0;
                for (int64_t i = 0; i <= t; ++i) {
                    if (!swa_oracle_allowed(t, i, w_loc, s))
                        continue;
                    const double *ki = k + ((b * L + i) * Hkv + h / group) * d;
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += qr[c] * ki[c];
                    lg[i] = scale * dot;
                    if (lg[i] > m)
                        m = lg[i];
                }
                for (int64_t i = 0; i <= t; ++i)
                    if (swa_oracle_allowed(t, i, w_loc, s))
                        sum += exp(lg[i] - m);
                lse[(b * (t_hi - t_lo) + (t - t_lo)) * Hq + h] = m + log(sum);
            }
    free(lg);
    return 0;
}

/* One decode row from an explicit set of cached positions.
 *   q: [Hq][d] for the query at position t.
 *   pos: [n] distinct absolute positions; k, v: [n][Hkv][d] their keys and values.
 * The entries whose position is in A(t) are kept (by the predicate), the others are
 * ignored, and out[h] = softmax-weighted sum over the kept entries for each q-head.
 * Returns the number of kept entries, or -1 on bad arguments / duplicate positions. */
static int cmp_i64(const void *a, const void *b)
{
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* 1 if two of pos[0..n-1] are equal, 0 if not, -1 if out of memory (a sorted copy, then
 * neighbours compared: n log n, so explicit sets of millions of entries stay cheap). */
static int has_duplicates(const int64_t *pos, int64_t n)
{
    int64_t *c = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    if (!c)
        return -1;
    memcpy(c, pos, (size_t)n * sizeof(int64_t));
    qsort(c, (size_t)n, sizeof(int64_t), cmp_i64);
    int dup = 0;
    for (int64_t i = 1; i < n && !dup; ++i)
        dup = c[i] == c[i - 1];
    free(c);
    return dup;
}

int64_t swa_oracle_decode_row(const double *q, const int64_t *pos, const double *k,
                              const double *v, int64_t n, int64_t t, int64_t Hq, int64_t Hkv,
                              int64_t d, int64_t w_loc, int64_t s, double scale, double *out)
{
    if (!q || !pos || !k || !v || !out || n < 1 || Hkv < 1 || Hq % Hkv != 0 || w_loc < 1 ||
        s < 0)
        return -1;
    if (has_duplicates(pos, n) != 0)
        return -1;
    const int64_t group = Hq / Hkv;
    double *lg = (double *)malloc((size_t)n * sizeof(double));
    if (!lg)
        return -1;
    int64_t kept = 0;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t kvh = h / group;
        const double *qh = q + h * d;
        double m = -INFINITY, den = 0.0;
        kept = 0;
        for (int64_t j = 0; j < n; ++j) {
            if (!swa_oracle_allowed(t, pos[j], w_loc, s))
                continue;
            const double *kj = k + (j * Hkv + kvh) * d;
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dot += qh[c] * kj[c];
            lg[j] = scale * dot;
            if (lg[j] > m)
                m = lg[j];
            ++kept;
        }
        double *xh = out + h * d;
        for (int64_t c = 0; c < d; ++c)
            xh[c] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (!swa_oracle_allowed(t, pos[j], w_loc, s))
                continue;
            lg[j] = exp(lg[j] - m);
            den += lg[j];
        }
        for (int64_t j = 0; j < n; ++j) {
            if (!swa_oracle_allowed(t, pos[j], w_loc, s))
                continue;
            const double pj = lg[j] / den;
            const double *vj = v + (j * Hkv + kvh) * d;
            for (int64_t c = 0; c < d; ++c)
                xh[c] += pj * vj[c];
        }
    }
    free(lg);
    return kept;
}

/* Plain simulation of a KV cache made of s pinned sink slots followed by a ring of
 * w_loc slots, after appending positions 0..n_appended-1 one at a time in order.
 * Position p goes to slot p when p < s, else to slot s + (p mod w_loc), replacing what
 * that slot held (the oldest ring entry).  slot_pos[j] receives the position held by
 * slot j, or -1 if nothing was ever written there.  Sources: page "从长文档摘要说起",
 * section "与 KV Cache 的配合：轮转替换策略" (evict the oldest entry, circular buffer
 * indexed modulo the window), and the first page's "64+4=68 tokens" deployment note
 * for the pinned sinks.  Returns 0, or -1 on bad arguments. */
int swa_oracle_ring_simulate(int64_t n_appended, int64_t w_loc, int64_t s, int64_t *slot_pos)
{
    if (!slot_pos || n_appended < 0 || w_loc < 1 || s < 0)
        return -1;
    for (int64_t j = 0; j < s + w_loc; ++j)
        slot_pos[j] = -1;
    for (int64_t p = 0; p < n_appended; ++p) {
        const int64_t slot = (p < s) ? p : s + (p % w_loc);
        slot_pos[slot] = p;
    }
    return 0;
}

typedef struct {
    const double *q, *k, *v;
    const int64_t *pos, *t;
    double *out;
    int64_t B, n, Hq, Hkv, d, w_loc, s;
    double scale;
    int64_t nthreads, tid, status;
} decode_job;

static void *decode_worker(void *arg)
{
    decode_job *j = (decode_job *)arg;
    j->status = 0;
    for (int64_t b = j->tid; b < j->B; b += j->nthreads) {
        const int64_t kept = swa_oracle_decode_row(
            j->q + b * j->Hq * j->d, j->pos, j->k + b * j->n * j->Hkv * j->d,
            j->v + b * j->n * j->Hkv * j->d, j->n, j->t[b], j->Hq, j->Hkv, j->d, j->w_loc, j->s,
            j->scale, j->out + b * j->Hq * j->d);
        if (kept < 0)
            j->status = -1;
    }
    return NULL;
}

/* Decode rows of a batch, one swa_oracle_decode_row per batch item, items spread over
 * threads.  q: [B][Hq][d]; pos: [n] shared candidate positions; k, v: [B][n][Hkv][d];
 * t: [B] query positions; out: [B][Hq][d].  Returns 0, or -1 if any row failed. */
int swa_oracle_decode_rows(const double *q, const int64_t *pos, const double *k, const double *v,
                           int64_t B, int64_t n, const int64_t *t, int64_t Hq, int64_t Hkv,
                           int64_t d, int64_t w_loc, int64_t s, double scale, double *out,
                           int nthreads)
{
    if (B < 1 || !t)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > B)
        nthreads = (int)B;
    decode_job *jobs = (decode_job *)calloc((size_t)nthreads, sizeof(decode_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        decode_job j = {q, k, v, pos, t, out, B, n, Hq, Hkv, d, w_loc, s, scale, nthreads, i, -3};
        jobs[i] = j;
        if (pthread_create(&th[i], NULL, decode_worker, &jobs[i]) != 0) {
            rc = -1;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(th[i], NULL);
        if (jobs[i].status != 0)
            rc = -1;
    }
    free(jobs);
    free(th);
    return rc;
}

/*
 * oracle.c -- plain fp64 CPU oracle (see oracle.h for what it computes and
 * where each definition comes from).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product library.
 *
 * Deliberately slow and literal: every mask entry is evaluated from the
 * element predicate, and attention visits every key of a row and skips the
 * masked ones (exp(-inf) = 0 contributes nothing to eq. 2's softmax).
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static int64_t iabs64(int64_t x) { return x < 0 ? -x : x; }

/* floor(log2(x)) for x >= 1, as bit length minus one. */
static int64_t floor_log2(int64_t x)
{
    int64_t r = -1;
    while (x > 0) {
        r++;
        x >>= 1;
    }
    return r;
}

/* Radial Attention, section 3, eq. 4.  With r = floor(log2(max(|i-j|, 1)))
 * an entry is kept when
 *   (a) 2^r <= s and |k - l| + 1 <= s / 2^r, or
 *   (b) |i - j| mod ceil(2^r / s) == 0 and k == l.
 * (a) is tested as (|k - l| + 1) * 2^r <= s, the same inequality multiplied
 * by 2^r > 0, so no real division is needed. */
static int keep_radial(int64_t s, int64_t q, int64_t t)
{
    int64_t i = q / s, k = q % s;
    int64_t j = t / s, l = t % s;
    int64_t delta = iabs64(i - j);
    int64_t r = floor_log2(delta > 1 ? delta : 1);
    int64_t p2 = (int64_t)1 << r;
    if (p2 <= s && (iabs64(k - l) + 1) * p2 <= s)
        return 1;
    int64_t stride = (p2 + s - 1) / s; /* ceil(2^r / s) */
    if (delta % stride == 0 && k == l)
        return 1;
    return 0;
}

/* Token radius neighbourhood on a (T, H, W) grid flattened t-h-w:
 * |dt| <= r_t and max(|dh|, |dw|) <= r_s. */
static int keep_radius3d(const orc_mask *m, int64_t q, int64_t t)
{
    int64_t hw = m->grid_h * m->grid_w;
    int64_t tq = q / hw, hq = (q % hw) / m->grid_w, wq = q % m->grid_w;
    int64_t tk = t / hw, hk = (t % hw) / m->grid_w, wk = t % m->grid_w;
    int64_t dh = iabs64(hq - hk), dw = iabs64(wq - wk);
    int64_t cheb = dh > dw ? dh : dw;
    return iabs64(tq - tk) <= m->r_t && cheb <= m->r_s;
}

/* Vera 1.1 temporal module, section 2.2: query frame i sees key frames
 * max(0, i - W + 1) .. i (causal AND window), all tokens of those frames. */
static int keep_swa(const orc_mask *m, int64_t q, int64_t t)
{
    int64_t i = q / m->s, j = t / m->s;
    int64_t lo = i - m->window + 1;
    if (lo < 0)
        lo = 0;
    return j >= lo && j <= i;
}

int orc_keep(const orc_mask *m, int64_t q, int64_t t)
{
    /* Sink: the keys of the first sink_frames frames are kept by every query
     * (the frame length is s for every family; RADIUS3D has s = H * W). */
    if (t / m->s < m->sink_frames)
        return 1;
    switch (m->kind) {
    case ORC_DENSE:
        return 1;
    case ORC_RADIAL:
        return keep_radial(m->s, q, t);
    case ORC_RADIUS3D:
        return keep_radius3d(m, q, t);
    case ORC_SWA:
        return keep_swa(m, q, t);
    default:
        return 0;
    }
}

/* Second block reading of Radial Attention section 6: the 128 x 128 blocks
 * themselves form a video of f frames with s / block blocks per frame, and
 * eq. 4 decides block (bq, bk) as it decides a token pair. */
int orc_keep_block_eq4(const orc_mask *m, int64_t bq, int64_t bk)
{
    int64_t sb = m->s / m->block;
    if (bk / sb < m->sink_frames)
        return 1;
    return keep_radial(sb, bq, bk);
}

void orc_block_keep(const orc_mask *m, uint8_t *out, int threads)
{
    int64_t n = m->f * m->s;
    int64_t nb = (n + m->block - 1) / m->block;
    if (m->granularity == ORC_BLOCK_EQ4) {
        for (int64_t bq = 0; bq < nb; bq++)
            for (int64_t bk = 0; bk < nb; bk++)
                out[bq * nb + bk] = (uint8_t)orc_keep_block_eq4(m, bq, bk);
        return;
    }
    int64_t *cnt = (int64_t *)malloc((size_t)(nb * nb) * sizeof(int64_t));
    orc_block_counts(m, cnt, threads);
    for (int64_t i = 0; i < nb * nb; i++)
        out[i] = cnt[i] > 0;
    free(cnt);
}

void orc_elem_matrix(const orc_mask *m, uint8_t *out)
{
    int64_t n = m->f * m->s;
    for (int64_t q = 0; q < n; q++)
        for (int64_t t = 0; t < n; t++)
            out[q * n + t] = (uint8_t)orc_keep(m, q, t);
}

/* ---- block counts (threaded over block rows) ---------------------------- */

typedef struct {
    const orc_mask *m;
    int64_t *out;
    int64_t row_begin, row_end, nb, n;
} count_job;

static void *count_worker(void *arg)
{
    count_job *j = (count_job *)arg;
    const int64_t bsz = j->m->block;
    for (int64_t bq = j->row_begin; bq < j->row_end; bq++) {
        for (int64_t bk = 0; bk < j->nb; bk++) {
            int64_t c = 0;
            for (int64_t q = bq * bsz; q < (bq + 1) * bsz && q < j->n; q++)
                for (int64_t t = bk * bsz; t < (bk + 1) * bsz && t < j->n; t++)
                    c += orc_keep(j->m, q, t);
            j->out[bq * j->nb + bk] = c;
        }
    }
    return NULL;
}

void orc_block_counts(const orc_mask *m, int64_t *out, int threads)
{
    int64_t n = m->f * m->s;
    int64_t nb = (n + m->block - 1) / m->block;
    if (threads < 1)
        threads = 1;
    if (threads > nb)
        threads = (int)nb;
    count_job *jobs = (count_job *)calloc((size_t)threads, sizeof(count_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int w = 0; w < threads; w++) {
        jobs[w].m = m;
        jobs[w].out = out;
        jobs[w].nb = nb;
        jobs[w].n = n;
        jobs[w].row_begin = nb * w / threads;
        jobs[w].row_end = nb * (w + 1) / threads;
        pthread_create(&tid[w], NULL, count_worker, &jobs[w]);
    }
    for (int w = 0; w < threads; w++)
        pthread_join(tid[w], NULL);
    free(jobs);
    free(tid);
}

typedef struct {
    const orc_mask *m;
    const int64_t *rows;
    int64_t *out;
    int64_t begin, end, nb, n;
} count_rows_job;

static void *count_rows_worker(void *arg)
{
    count_rows_job *j = (count_rows_job *)arg;
    const int64_t bsz = j->m->block;
    for (int64_t i = j->begin; i < j->end; i++) {
        int64_t bq = j->rows[i];
        for (int64_t bk = 0; bk < j->nb; bk++) {
            int64_t c = 0;
            for (int64_t q = bq * bsz; q < (bq + 1) * bsz && q < j->n; q++)
                for (int64_t t = bk * bsz; t < (bk + 1) * bsz && t < j->n; t++)
                    c += orc_keep(j->m, q, t);
            j->out[i * j->nb + bk] = c;
        }
    }
    return NULL;
}

void orc_block_counts_rows(const orc_mask *m, const int64_t *rows, int64_t nrows, int64_t *out,
                           int threads)
{
    int64_t n = m->f * m->s;
    int64_t nb = (n + m->block - 1) / m->block;
    if (threads < 1)
        threads = 1;
    if (threads > nrows)
        threads = nrows > 0 ? (int)nrows : 1;
    count_rows_job *jobs = (count_rows_job *)calloc((size_t)threads, sizeof(count_rows_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int w = 0; w < threads; w++) {
        jobs[w].m = m;
        jobs[w].rows = rows;
        jobs[w].out = out;
        jobs[w].nb = nb;
        jobs[w].n = n;
        jobs[w].begin = nrows * w / threads;
        jobs[w].end = nrows * (w + 1) / threads;
        pthread_create(&tid[w], NULL, count_rows_worker, &jobs[w]);
    }
    for (int w = 0; w < threads; w++)
        pthread_join(tid[w], NULL);
    free(jobs);
    free(tid);
}

int64_t orc_kept_elements(const orc_mask *m, int threads)
{
    int64_t n = m->f * m->s;
    int64_t nb = (n + m->block - 1) / m->block;
    int64_t *cnt = (int64_t *)malloc((size_t)(nb * nb) * sizeof(int64_t));
    orc_block_counts(m, cnt, threads);
    int64_t tot = 0;
    for (int64_t i = 0; i < nb * nb; i++)
        tot += cnt[i];
    free(cnt);
    return tot;
}

void orc_block_bits128(const orc_mask *m, int64_t qb, int64_t kb, uint32_t *out)
{
    int64_t n = m->f * m->s;
    memset(out, 0, 128 * 4 * sizeof(uint32_t));
    for (int64_t r = 0; r < 128; r++) {
        int64_t q = qb * 128 + r;
        if (q >= n)
            continue;
        for (int64_t c = 0; c < 128; c++) {
            int64_t t = kb * 128 + c;
            if (t < n && orc_keep(m, q, t))
                out[r * 4 + c / 32] |= (uint32_t)1 << (c % 32);
        }
    }
}

/* ---- attention ---------------------------------------------------------- */

static double load_value(int dtype, const void *base, int64_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    /* bfloat16 is the upper half of an IEEE binary32: widen by shifting. */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    int dtype;
    const void *q, *k, *v;
    int64_t H, n, d;
    const orc_mask *mask;
    const uint8_t *block_keep;
    double scale;
    const int64_t *rows;
    int64_t begin, end;
    double *o_out, *lse_out;
} attn_job;

static int key_kept(const attn_job *j, int64_t q, int64_t t)
{
    if (j->mask->granularity == ORC_BLOCK_EQ4)
        return orc_keep_block_eq4(j->mask, q / j->mask->block, t / j->mask->block);
    if (j->mask->granularity == ORC_BLOCK_ANY) {
        int64_t nb = (j->n + j->mask->block - 1) / j->mask->block;
        return j->block_keep[(q / j->mask->block) * nb + t / j->mask->block] != 0;
    }
    return orc_keep(j->mask, q, t);
}

static void *attn_worker(void *arg)
{
    attn_job *j = (attn_job *)arg;
    const int64_t n = j->n, d = j->d;
    double *score = (double *)malloc((size_t)n * sizeof(double));
    double *qrow = (double *)malloc((size_t)d * sizeof(double));
    for (int64_t r = j->begin; r < j->end; r++) {
        int64_t b = j->rows[3 * r], h = j->rows[3 * r + 1], q = j->rows[3 * r + 2];
        int64_t head = (b * j->H + h) * n * d; /* element offset of [b, h, 0, 0] */
        double *o = j->o_out + r * d;
        for (int64_t x = 0; x < d; x++) {
            qrow[x] = load_value(j->dtype, j->q, head + q * d + x);
            o[x] = 0.0;
        }
        /* eq. 2: scaled scores of the kept keys; the max makes exp stable. */
        double mx = -INFINITY;
        for (int64_t t = 0; t < n; t++) {
            if (!key_kept(j, q, t)) {
                score[t] = -INFINITY;
                continue;
            }
            double acc = 0.0;
            for (int64_t x = 0; x < d; x++)
                acc += qrow[x] * load_value(j->dtype, j->k, head + t * d + x);
            score[t] = acc * j->scale;
            if (score[t] > mx)
                mx = score[t];
        }
        if (mx == -INFINITY) {
            j->lse_out[r] = -INFINITY;
            continue;
        }
        double denom = 0.0;
        for (int64_t t = 0; t < n; t++) {
            if (score[t] == -INFINITY)
                continue;
            double p = exp(score[t] - mx);
            denom += p;
            for (int64_t x = 0; x < d; x++)
                o[x] += p * load_value(j->dtype, j->v, head + t * d + x);
        }
        for (int64_t x = 0; x < d; x++)
            o[x] /= denom;
        j->lse_out[r] = mx + log(denom);
    }
    free(score);
    free(qrow);
    return NULL;
}

void orc_row_counts(const orc_mask *m, const uint8_t *block_keep, const int64_t *rows, int64_t nrows,
                    int64_t *out)
{
    attn_job j;
    memset(&j, 0, sizeof j);
    j.n = m->f * m->s;
    j.mask = m;
    j.block_keep = block_keep;
    for (int64_t r = 0; r < nrows; r++) {
        int64_t c = 0;
        for (int64_t t = 0; t < j.n; t++)
            c += key_kept(&j, rows[r], t);
        out[r] = c;
    }
}

void orc_attention_rows(int dtype, const void *q, const void *k, const void *v,
                        int64_t B, int64_t H, int64_t n, int64_t d,
                        const orc_mask *mask, const uint8_t *block_keep,
                        double scale, const int64_t *rows, int64_t nrows,
                        double *o_out, double *lse_out, int threads)
{
    (void)B;
    if (threads < 1)
        threads = 1;
    if (threads > nrows)
        threads = nrows > 0 ? (int)nrows : 1;
    attn_job *jobs = (attn_job *)calloc((size_t)threads, sizeof(attn_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int w = 0; w < threads; w++) {
        attn_job *j = &jobs[w];
        j->dtype = dtype;
        j->q = q;
        j->k = k;
        j->v = v;
        j->H = H;
        j->n = n;
        j->d = d;
        j->mask = mask;
        j->block_keep = block_keep;
        j->scale = scale;
        j->rows = rows;
        j->begin = nrows * w / threads;
        j->end = nrows * (w + 1) / threads;
        j->o_out = o_out;
        j->lse_out = lse_out;
        pthread_create(&tid[w], NULL, attn_worker, j);
    }
    for (int w = 0; w < threads; w++)
        pthread_join(tid[w], NULL);
    free(jobs);
    free(tid);
}

/* ---- backward ------------------------------------------------------------ */

/* Softmax row of query q (scaled scores, masked keys -> -inf) and the row's
 * dP entries: p[t] (0 for masked keys), dp[t] = dO[q] . V[t].  Returns
 * rowsum(p o dp). */
static double softmax_row(const attn_job *j, const void *dout, int64_t head, int64_t q, double *qrow,
                          double *p, double *dp)
{
    const int64_t n = j->n, d = j->d;
    for (int64_t x = 0; x < d; x++)
        qrow[x] = load_value(j->dtype, j->q, head + q * d + x);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; t++) {
        if (!key_kept(j, q, t)) {
            p[t] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int64_t x = 0; x < d; x++)
            acc += qrow[x] * load_value(j->dtype, j->k, head + t * d + x);
        p[t] = acc * j->scale;
        if (p[t] > mx)
            mx = p[t];
    }
    double denom = 0.0;
    for (int64_t t = 0; t < n; t++) {
        p[t] = (p[t] == -INFINITY || mx == -INFINITY) ? 0.0 : exp(p[t] - mx);
        denom += p[t];
    }
    double delta = 0.0;
    for (int64_t t = 0; t < n; t++) {
        if (denom > 0.0)
            p[t] /= denom;
        dp[t] = 0.0;
        if (p[t] == 0.0 && !key_kept(j, q, t))
            continue;
        double acc = 0.0;
        for (int64_t x = 0; x < d; x++)
            acc += load_value(j->dtype, dout, head + q * d + x) * load_value(j->dtype, j->v, head + t * d + x);
        dp[t] = acc;
        delta += p[t] * acc;
    }
    return delta;
}

typedef struct {
    attn_job base;
    const void *dout;
    const int64_t *rows;
    int64_t begin, end;
    double *dq, *dk, *dv;
} bwd_job;

/* dQ rows: dQ[q] = scale sum_t dS[q, t] K[t]. */
static void *bwd_q_worker(void *arg)
{
    bwd_job *w = (bwd_job *)arg;
    const attn_job *j = &w->base;
    const int64_t n = j->n, d = j->d;
    double *p = (double *)malloc((size_t)n * sizeof(double));
    double *dp = (double *)malloc((size_t)n * sizeof(double));
    double *qrow = (double *)malloc((size_t)d * sizeof(double));
    for (int64_t r = w->begin; r < w->end; r++) {
        int64_t b = w->rows[3 * r], h = w->rows[3 * r + 1], q = w->rows[3 * r + 2];
        int64_t head = (b * j->H + h) * n * d;
        double delta = softmax_row(j, w->dout, head, q, qrow, p, dp);
        double *out = w->dq + r * d;
        for (int64_t x = 0; x < d; x++)
            out[x] = 0.0;
        for (int64_t t = 0; t < n; t++) {
            double ds = p[t] * (dp[t] - delta);
            if (ds == 0.0)
                continue;
            for (int64_t x = 0; x < d; x++)
                out[x] += ds * load_value(j->dtype, j->k, head + t * d + x);
        }
        for (int64_t x = 0; x < d; x++)
            out[x] *= j->scale;
    }
    free(p);
    free(dp);
    free(qrow);
    return NULL;
}

/* dK/dV rows of the listed keys, one (b, h) at a time: every query of the
 * head contributes dV[t] += P[q, t] dO[q] and dK[t] += scale dS[q, t] Q[q].
 * Threads split the queries; each keeps private sums that are added at
 * the end (in a fixed order). */
typedef struct {
    attn_job base;
    const void *dout;
    int64_t head, q0, q1;
    const int64_t *keys;  /* key indices of this head's listed rows */
    int64_t nkeys;
    double *dk, *dv;      /* nkeys x d private sums */
} bwd_kv_job;

static void *bwd_kv_worker(void *arg)
{
    bwd_kv_job *w = (bwd_kv_job *)arg;
    const attn_job *j = &w->base;
    const int64_t n = j->n, d = j->d;
    double *p = (double *)malloc((size_t)n * sizeof(double));
    double *dp = (double *)malloc((size_t)n * sizeof(double));
    double *qrow = (double *)malloc((size_t)d * sizeof(double));
    for (int64_t q = w->q0; q < w->q1; q++) {
        int any = 0;
        for (int64_t i = 0; i < w->nkeys && !any; i++)
            any = key_kept(j, q, w->keys[i]);
        if (!any)
            continue;
        double delta = softmax_row(j, w->dout, w->head, q, qrow, p, dp);
        for (int64_t i = 0; i < w->nkeys; i++) {
            int64_t t = w->keys[i];
            if (p[t] == 0.0 && dp[t] == 0.0)
                continue;
            double ds = p[t] * (dp[t] - delta) * j->scale;
            for (int64_t x = 0; x < d; x++) {
                w->dv[i * d + x] += p[t] * load_value(j->dtype, w->dout, w->head + q * d + x);
                w->dk[i * d + x] += ds * qrow[x];
            }
        }
    }
    free(p);
    free(dp);
    free(qrow);
    return NULL;
}

void orc_attention_bwd_rows(int dtype, const void *q, const void *k, const void *v, const void *dout,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            const orc_mask *mask, const uint8_t *block_keep, double scale,
                            const int64_t *q_rows, int64_t nq, double *dq_out,
                            const int64_t *k_rows, int64_t nk, double *dk_out, double *dv_out,
                            int threads)
{
    (void)B;
    if (threads < 1)
        threads = 1;
    attn_job base;
    memset(&base, 0, sizeof base);
    base.dtype = dtype;
    base.q = q;
    base.k = k;
    base.v = v;
    base.H = H;
    base.n = n;
    base.d = d;
    base.mask = mask;
    base.block_keep = block_keep;
    base.scale = scale;
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (nq > 0) {
        int tq = threads > nq ? (int)nq : threads;
        bwd_job *jobs = (bwd_job *)calloc((size_t)tq, sizeof(bwd_job));
        for (int w = 0; w < tq; w++) {
            jobs[w].base = base;
            jobs[w].dout = dout;
            jobs[w].rows = q_rows;
            jobs[w].begin = nq * w / tq;
            jobs[w].end = nq * (w + 1) / tq;
            jobs[w].dq = dq_out;
            pthread_create(&tid[w], NULL, bwd_q_worker, &jobs[w]);
        }
        for (int w = 0; w < tq; w++)
            pthread_join(tid[w], NULL);
        free(jobs);
    }
    /* dK/dV: group the listed rows by head */
    for (int64_t i = 0; i < nk * d; i++) {
        dk_out[i] = 0.0;
        dv_out[i] = 0.0;
    }
    char *done = (char *)calloc((size_t)(nk > 0 ? nk : 1), 1);
    int64_t *idx = (int64_t *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(int64_t));
    int64_t *keys = (int64_t *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(int64_t));
    for (int64_t r0 = 0; r0 < nk; r0++) {
        if (done[r0])
            continue;
        int64_t b = k_rows[3 * r0], h = k_rows[3 * r0 + 1];
        int64_t cnt = 0;
        for (int64_t r = r0; r < nk; r++)
            if (!done[r] && k_rows[3 * r] == b && k_rows[3 * r + 1] == h) {
                done[r] = 1;
                idx[cnt] = r;
                keys[cnt] = k_rows[3 * r + 2];
                cnt++;
            }
        bwd_kv_job *jobs = (bwd_kv_job *)calloc((size_t)threads, sizeof(bwd_kv_job));
        for (int w = 0; w < threads; w++) {
            jobs[w].base = base;
            jobs[w].dout = dout;
            jobs[w].head = (b * H + h) * n * d;
            jobs[w].q0 = n * w / threads;
            jobs[w].q1 = n * (w + 1) / threads;
            jobs[w].keys = keys;
            jobs[w].nkeys = cnt;
            jobs[w].dk = (double *)calloc((size_t)(cnt * d), sizeof(double));
            jobs[w].dv = (double *)calloc((size_t)(cnt * d), sizeof(double));
            pthread_create(&tid[w], NULL, bwd_kv_worker, &jobs[w]);
        }
        for (int w = 0; w < threads; w++)
            pthread_join(tid[w], NULL);
        for (int w = 0; w < threads; w++) {
            for (int64_t i = 0; i < cnt; i++)
                for (int64_t x = 0; x < d; x++) {
                    dk_out[idx[i] * d + x] += jobs[w].dk[i * d + x];
                    dv_out[idx[i] * d + x] += jobs[w].dv[i * d + x];
                }
            free(jobs[w].dk);
            free(jobs[w].dv);
        }
        free(jobs);
    }
    free(done);
    free(idx);
    free(keys);
    free(tid);
}

/* ---- SALAD linear branch ------------------------------------------------- */

typedef struct {
    int dtype;
    const void *q, *k, *v;
    int64_t H, n, d;
    double eps;
    const int64_t *rows;
    int64_t begin, end;
    double *o_out;
} lin_job;

static double relu(double x) { return x > 0.0 ? x : 0.0; }

static void *lin_worker(void *arg)
{
    lin_job *j = (lin_job *)arg;
    const int64_t n = j->n, d = j->d;
    double *fq = (double *)malloc((size_t)d * sizeof(double));
    for (int64_t r = j->begin; r < j->end; r++) {
        int64_t b = j->rows[3 * r], h = j->rows[3 * r + 1], q = j->rows[3 * r + 2];
        int64_t head = (b * j->H + h) * n * d;
        double *o = j->o_out + r * d;
        for (int64_t x = 0; x < d; x++) {
            fq[x] = relu(load_value(j->dtype, j->q, head + q * d + x));
            o[x] = 0.0;
        }
        double wsum = 0.0;
        for (int64_t t = 0; t < n; t++) {
            double w = 0.0;
            for (int64_t x = 0; x < d; x++)
                w += fq[x] * relu(load_value(j->dtype, j->k, head + t * d + x));
            if (w == 0.0)
                continue;
            wsum += w;
            for (int64_t x = 0; x < d; x++)
                o[x] += w * load_value(j->dtype, j->v, head + t * d + x);
        }
        for (int64_t x = 0; x < d; x++)
            o[x] /= wsum + j->eps;
    }
    free(fq);
    return NULL;
}

void orc_linear_attention_rows(int dtype, const void *q, const void *k, const void *v, int64_t B, int64_t H,
                               int64_t n, int64_t d, double eps, const int64_t *rows, int64_t nrows,
                               double *o_out, int threads)
{
    (void)B;
    if (threads < 1)
        threads = 1;
    if (threads > nrows)
        threads = nrows > 0 ? (int)nrows : 1;
    lin_job *jobs = (lin_job *)calloc((size_t)threads, sizeof(lin_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int w = 0; w < threads; w++) {
        lin_job *j = &jobs[w];
        j->dtype = dtype;
        j->q = q;
        j->k = k;
        j->v = v;
        j->H = H;
        j->n = n;
        j->d = d;
        j->eps = eps;
        j->rows = rows;
        j->begin = nrows * w / threads;
        j->end = nrows * (w + 1) / threads;
        j->o_out = o_out;
        pthread_create(&tid[w], NULL, lin_worker, j);
    }
    for (int w = 0; w < threads; w++)
        pthread_join(tid[w], NULL);
    free(jobs);
    free(tid);
}

/* ---- SALAD gate and output ------------------------------------------------ */

typedef struct {
    int dtype;
    const void *x, *w;
    double bias;
    int64_t N, C;
    int64_t begin, end; /* samples b */
    double *g_out;
} gate_job;

static void *gate_worker(void *arg)
{
    gate_job *j = (gate_job *)arg;
    for (int64_t b = j->begin; b < j->end; b++) {
        double sum = 0.0;
        for (int64_t n = 0; n < j->N; n++) {
            double z = j->bias;
            for (int64_t c = 0; c < j->C; c++)
                z += load_value(j->dtype, j->x, (b * j->N + n) * j->C + c) * load_value(j->dtype, j->w, c);
            sum += 1.0 / (1.0 + exp(-z));
        }
        j->g_out[b] = sum / (double)j->N;
    }
    return NULL;
}

void orc_salad_gate(int dtype, const void *x, const void *w, double bias, int64_t B, int64_t N, int64_t C,
                    double *g_out, int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > B)
        threads = B > 0 ? (int)B : 1;
    gate_job *jobs = (gate_job *)calloc((size_t)threads, sizeof(gate_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int t = 0; t < threads; t++) {
        gate_job *j = &jobs[t];
        j->dtype = dtype;
        j->x = x;
        j->w = w;
        j->bias = bias;
        j->N = N;
        j->C = C;
        j->begin = B * t / threads;
        j->end = B * (t + 1) / threads;
        j->g_out = g_out;
        pthread_create(&tid[t], NULL, gate_worker, j);
    }
    for (int t = 0; t < threads; t++)
        pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
}

typedef struct {
    int dtype;
    const void *os, *ol, *w;
    const double *bias, *g;
    int64_t H, N, d;
    const int64_t *rows;
    int64_t begin, end;
    double *out;
} sout_job;

static void *sout_worker(void *arg)
{
    sout_job *j = (sout_job *)arg;
    const int64_t H = j->H, N = j->N, d = j->d, C = H * d;
    double *in = (double *)malloc((size_t)C * sizeof(double));
    for (int64_t r = j->begin; r < j->end; r++) {
        const int64_t b = j->rows[2 * r], n = j->rows[2 * r + 1];
        /* channel c of token n: head c / d, element c % d */
        for (int64_t c = 0; c < C; c++)
            in[c] = load_value(j->dtype, j->ol, ((b * H + c / d) * N + n) * d + c % d);
        for (int64_t co = 0; co < C; co++) {
            double acc = 0.0;
            for (int64_t c = 0; c < C; c++)
                acc += in[c] * load_value(j->dtype, j->w, co * C + c);
            if (j->bias)
                acc += j->bias[co];
            j->out[r * C + co] =
                load_value(j->dtype, j->os, ((b * H + co / d) * N + n) * d + co % d) + j->g[b] * acc;
        }
    }
    free(in);
    return NULL;
}

void orc_salad_output_rows(int dtype, const void *o_sparse, const void *o_lin, const void *w, const double *bias,
                           const double *g, int64_t B, int64_t H, int64_t N, int64_t d, const int64_t *rows,
                           int64_t nrows, double *out, int threads)
{
    (void)B;
    if (threads < 1)
        threads = 1;
    if (threads > nrows)
        threads = nrows > 0 ? (int)nrows : 1;
    sout_job *jobs = (sout_job *)calloc((size_t)threads, sizeof(sout_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    for (int t = 0; t < threads; t++) {
        sout_job *j = &jobs[t];
        j->dtype = dtype;
        j->os = o_sparse;
        j->ol = o_lin;
        j->w = w;
        j->bias = bias;
        j->g = g;
        j->H = H;
        j->N = N;
        j->d = d;
        j->rows = rows;
        j->begin = nrows * t / threads;
        j->end = nrows * (t + 1) / threads;
        j->out = out;
        pthread_create(&tid[t], NULL, sout_worker, j);
    }
    for (int t = 0; t < threads; t++)
        pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
}

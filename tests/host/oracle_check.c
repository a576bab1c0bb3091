/*
 * Calls every entry point of the C oracle (oracle/oracle.c) on small inputs,
 * meant to run under AddressSanitizer and UndefinedBehaviorSanitizer, and
 * checks closed forms that each result must meet:
 *   - the dense element matrix, the block counts (all blocks and listed
 *     rows), the kept-element total, the kept-block matrix, the 128-bit block
 *     rows and the per-row key counts all agree with orc_keep, element by
 *     element, for every mask family (with and without sink frames);
 *   - the eq. 4 block reading agrees with orc_keep_block_eq4;
 *   - attention with a constant V returns that constant on every row that
 *     keeps a key, and with Q = 0 its LSE is ln(kept keys) (fp32 and bf16
 *     inputs); rows without keys give O = 0 and LSE = -inf;
 *   - the gradients over every query and key of a head satisfy
 *     sum_keys dV = sum_queries dO (rows that keep a key) and sum_keys dK = 0;
 *   - the linear branch returns a constant V scaled by S / (S + eps);
 *   - the SALAD gate of w = 0 is sigmoid(bias); the SALAD output with g = 0
 *     is the sparse branch in the merged-head layout.
 * Exit status 0 when every check holds; the first violation exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int g_checks = 0;

#define CHECK(cond, ...)                                                                \
    do {                                                                                \
        ++g_checks;                                                                     \
        if (!(cond)) {                                                                  \
            fprintf(stderr, "%s:%d: check failed: %s\n  ", __FILE__, __LINE__, #cond);  \
            fprintf(stderr, __VA_ARGS__);                                               \
            fprintf(stderr, "\n");                                                      \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;

static double urand(void) /* xorshift64*, uniform in [-1, 1) */
{
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return (double)((g_rng * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static uint16_t to_bf16(float x) /* round to nearest even (finite inputs) */
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *xcalloc(size_t n, size_t size)
{
    void *p = calloc(n ? n : 1, size);
    if (p == NULL) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void check_mask(const orc_mask *m, const char *what)
{
    const int64_t n = m->f * m->s, blk = m->block, nb = (n + blk - 1) / blk;
    uint8_t *el = xcalloc((size_t)(n * n), 1);
    orc_elem_matrix(m, el);
    int64_t total = 0;
    for (int64_t q = 0; q < n; ++q)
        for (int64_t t = 0; t < n; ++t) {
            CHECK(el[q * n + t] == (orc_keep(m, q, t) != 0), "%s: element (%lld, %lld)", what, (long long)q,
                  (long long)t);
            total += el[q * n + t];
        }
    CHECK(orc_kept_elements(m, 3) == total, "%s: kept elements", what);

    int64_t *cnt = xcalloc((size_t)(nb * nb), sizeof(int64_t));
    orc_block_counts(m, cnt, 2);
    for (int64_t bq = 0; bq < nb; ++bq)
        for (int64_t bk = 0; bk < nb; ++bk) {
            int64_t c = 0;
            for (int64_t q = bq * blk; q < n && q < (bq + 1) * blk; ++q)
                for (int64_t t = bk * blk; t < n && t < (bk + 1) * blk; ++t)
                    c += el[q * n + t];
            CHECK(cnt[bq * nb + bk] == c, "%s: block (%lld, %lld) count", what, (long long)bq, (long long)bk);
        }
    int64_t rows[3] = {nb - 1, 0, nb / 2};
    int64_t *crow = xcalloc((size_t)(3 * nb), sizeof(int64_t));
    orc_block_counts_rows(m, rows, 3, crow, 2);
    for (int i = 0; i < 3; ++i)
        for (int64_t bk = 0; bk < nb; ++bk)
            CHECK(crow[i * nb + bk] == cnt[rows[i] * nb + bk], "%s: listed block row %d", what, i);

    orc_mask me = *m;
    me.granularity = ORC_ELEMENT;
    uint8_t *keep = xcalloc((size_t)(nb * nb), 1);
    orc_block_keep(&me, keep, 2);
    for (int64_t b = 0; b < nb * nb; ++b)
        CHECK(keep[b] == (cnt[b] > 0), "%s: kept block %lld", what, (long long)b);

    int64_t *qs = xcalloc((size_t)n, sizeof(int64_t)), *rc = xcalloc((size_t)n, sizeof(int64_t));
    for (int64_t q = 0; q < n; ++q)
        qs[q] = n - 1 - q;
    orc_row_counts(&me, NULL, qs, n, rc);
    for (int64_t i = 0; i < n; ++i) {
        int64_t c = 0;
        for (int64_t t = 0; t < n; ++t)
            c += el[qs[i] * n + t];
        CHECK(rc[i] == c, "%s: row %lld key count", what, (long long)qs[i]);
    }
    if (blk == 128) {
        uint32_t bits[128 * 4];
        for (int64_t bq = 0; bq < nb; ++bq)
            for (int64_t bk = 0; bk < nb; ++bk) {
                orc_block_bits128(m, bq, bk, bits);
                for (int r = 0; r < 128; ++r)
                    for (int c = 0; c < 128; ++c) {
                        const int64_t q = bq * 128 + r, t = bk * 128 + c;
                        const int want = q < n && t < n ? el[q * n + t] : 0;
                        CHECK((int)((bits[r * 4 + c / 32] >> (c % 32)) & 1u) == want, "%s: bit (%lld, %lld)", what,
                              (long long)q, (long long)t);
                    }
            }
    }
    free(el);
    free(cnt);
    free(crow);
    free(keep);
    free(qs);
    free(rc);
}

static void check_eq4(void)
{
    orc_mask m = {ORC_RADIAL, ORC_BLOCK_EQ4, 6, 256, 128, 0, 0, 0, 0, 0, 1};
    const int64_t nb = 6 * 256 / 128;
    uint8_t *keep = xcalloc((size_t)(nb * nb), 1);
    orc_block_keep(&m, keep, 2);
    for (int64_t bq = 0; bq < nb; ++bq)
        for (int64_t bk = 0; bk < nb; ++bk)
            CHECK(keep[bq * nb + bk] == (orc_keep_block_eq4(&m, bq, bk) != 0), "eq4 block (%lld, %lld)",
                  (long long)bq, (long long)bk);
    free(keep);
}

/* Attention closed forms on one mask, both input dtypes. */
static void check_attention(const orc_mask *m, const char *what)
{
    const int64_t B = 1, H = 2, n = m->f * m->s, d = 16, total = B * H * n * d;
    float *qf = xcalloc((size_t)total, 4), *kf = xcalloc((size_t)total, 4), *vf = xcalloc((size_t)total, 4);
    uint16_t *qb = xcalloc((size_t)total, 2), *kb = xcalloc((size_t)total, 2), *vb = xcalloc((size_t)total, 2);
    for (int64_t i = 0; i < total; ++i) {
        qf[i] = 0.f;
        kf[i] = (float)urand();
        vf[i] = 0.75f; /* exact in bf16 */
        qb[i] = to_bf16(qf[i]);
        kb[i] = to_bf16(kf[i]);
        vb[i] = to_bf16(vf[i]);
    }
    int64_t *rows = xcalloc((size_t)(3 * B * H * n), sizeof(int64_t)), *qs = xcalloc((size_t)n, sizeof(int64_t));
    int64_t nr = 0;
    for (int64_t h = 0; h < H; ++h)
        for (int64_t q = 0; q < n; ++q) {
            rows[3 * nr] = 0;
            rows[3 * nr + 1] = h;
            rows[3 * nr + 2] = q;
            ++nr;
        }
    for (int64_t q = 0; q < n; ++q)
        qs[q] = q;
    int64_t *cnt = xcalloc((size_t)n, sizeof(int64_t));
    orc_row_counts(m, NULL, qs, n, cnt);
    double *o = xcalloc((size_t)(nr * d), sizeof(double)), *lse = xcalloc((size_t)nr, sizeof(double));
    for (int dt = 0; dt < 2; ++dt) {
        orc_attention_rows(dt, dt ? (void *)qb : (void *)qf, dt ? (void *)kb : (void *)kf, dt ? (void *)vb : (void *)vf,
                           B, H, n, d, m, NULL, 0.25, rows, nr, o, lse, 3);
        for (int64_t r = 0; r < nr; ++r) {
            const int64_t q = rows[3 * r + 2];
            if (cnt[q] == 0) {
                CHECK(isinf(lse[r]) && lse[r] < 0, "%s: empty row %lld LSE", what, (long long)q);
                for (int64_t e = 0; e < d; ++e)
                    CHECK(o[r * d + e] == 0.0, "%s: empty row %lld O", what, (long long)q);
            } else {
                CHECK(fabs(lse[r] - log((double)cnt[q])) < 1e-12, "%s: row %lld LSE %g, want ln %lld", what,
                      (long long)q, lse[r], (long long)cnt[q]);
                for (int64_t e = 0; e < d; ++e)
                    CHECK(fabs(o[r * d + e] - 0.75) < 1e-12, "%s: row %lld O[%lld] = %g", what, (long long)q,
                          (long long)e, o[r * d + e]);
            }
        }
    }

    /* gradients over a whole head: random q, k, v, dO in fp32 */
    float *dof = xcalloc((size_t)total, 4);
    for (int64_t i = 0; i < total; ++i) {
        qf[i] = (float)urand();
        vf[i] = (float)urand();
        dof[i] = (float)urand();
    }
    int64_t *hrows = xcalloc((size_t)(3 * n), sizeof(int64_t));
    for (int64_t q = 0; q < n; ++q) {
        hrows[3 * q] = 0;
        hrows[3 * q + 1] = 1;
        hrows[3 * q + 2] = q;
    }
    double *dq = xcalloc((size_t)(n * d), sizeof(double)), *dk = xcalloc((size_t)(n * d), sizeof(double)),
           *dv = xcalloc((size_t)(n * d), sizeof(double));
    orc_attention_bwd_rows(ORC_F32, qf, kf, vf, dof, B, H, n, d, m, NULL, 0.25, hrows, n, dq, hrows, n, dk, dv, 3);
    for (int64_t e = 0; e < d; ++e) {
        double sdv = 0.0, sdo = 0.0, sdk = 0.0, mag = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            sdv += dv[t * d + e];
            sdk += dk[t * d + e];
            mag += fabs(dk[t * d + e]);
        }
        for (int64_t q = 0; q < n; ++q)
            if (cnt[q] > 0)
                sdo += dof[((0 * H + 1) * n + q) * d + e];
        CHECK(fabs(sdv - sdo) < 1e-9, "%s: sum dV %g, sum dO %g (dim %lld)", what, sdv, sdo, (long long)e);
        CHECK(fabs(sdk) < 1e-9 * (1.0 + mag), "%s: sum dK %g (dim %lld)", what, sdk, (long long)e);
        for (int64_t q = 0; q < n; ++q)
            CHECK(isfinite(dq[q * d + e]), "%s: dQ row %lld", what, (long long)q);
    }

    /* linear branch with constant V: O = v * S / (S + eps) */
    for (int64_t i = 0; i < total; ++i) {
        qf[i] = (float)fabs(urand()) + 0.01f;
        kf[i] = (float)fabs(urand()) + 0.01f;
        vf[i] = -1.5f;
    }
    orc_linear_attention_rows(ORC_F32, qf, kf, vf, B, H, n, d, 1e-3, rows, nr, o, 2);
    for (int64_t r = 0; r < nr; ++r) {
        const int64_t h = rows[3 * r + 1], q = rows[3 * r + 2];
        double S = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            double w = 0.0;
            for (int64_t e = 0; e < d; ++e)
                w += (double)qf[((0 * H + h) * n + q) * d + e] * (double)kf[((0 * H + h) * n + t) * d + e];
            S += w;
        }
        for (int64_t e = 0; e < d; ++e)
            CHECK(fabs(o[r * d + e] - (-1.5) * S / (S + 1e-3)) < 1e-9, "%s: linear row %lld", what, (long long)q);
    }

    free(qf), free(kf), free(vf), free(qb), free(kb), free(vb), free(dof);
    free(rows), free(qs), free(cnt), free(o), free(lse), free(hrows), free(dq), free(dk), free(dv);
}

static void check_salad(void)
{
    const int64_t B = 2, H = 3, N = 20, d = 8, C = H * d;
    float *x = xcalloc((size_t)(B * N * C), 4), *w = xcalloc((size_t)C, 4);
    for (int64_t i = 0; i < B * N * C; ++i)
        x[i] = (float)urand();
    double g[2];
    orc_salad_gate(ORC_F32, x, w, 0.3, B, N, C, g, 2);
    for (int b = 0; b < 2; ++b)
        CHECK(fabs(g[b] - 1.0 / (1.0 + exp(-0.3))) < 1e-15, "gate %d = %g", b, g[b]);

    float *os = xcalloc((size_t)(B * H * N * d), 4), *ol = xcalloc((size_t)(B * H * N * d), 4),
          *wp = xcalloc((size_t)(C * C), 4);
    for (int64_t i = 0; i < B * H * N * d; ++i) {
        os[i] = (float)urand();
        ol[i] = (float)urand();
    }
    for (int64_t i = 0; i < C * C; ++i)
        wp[i] = (float)urand();
    double bias[24], zero[2] = {0.0, 0.0}, out[3 * 24];
    for (int i = 0; i < 24; ++i)
        bias[i] = urand();
    int64_t rows[6] = {1, 19, 0, 0, 1, 7};
    orc_salad_output_rows(ORC_F32, os, ol, wp, bias, zero, B, H, N, d, rows, 3, out, 2);
    for (int r = 0; r < 3; ++r)
        for (int64_t c = 0; c < C; ++c) {
            const int64_t b = rows[2 * r], t = rows[2 * r + 1];
            const double want = os[((b * H + c / d) * N + t) * d + c % d];
            CHECK(out[r * C + c] == want, "salad output row %d channel %lld", r, (long long)c);
        }
    free(x), free(w), free(os), free(ol), free(wp);
}

int main(void)
{
    /* small instances of every family: kind, granularity, f, s, block, grid_h, grid_w, r_t, r_s, window, sink */
    const orc_mask masks[] = {
        {ORC_RADIAL, ORC_ELEMENT, 6, 20, 16, 0, 0, 0, 0, 0, 0},
        {ORC_RADIAL, ORC_ELEMENT, 9, 12, 32, 0, 0, 0, 0, 0, 2},
        {ORC_RADIAL, ORC_ELEMENT, 4, 80, 128, 0, 0, 0, 0, 0, 0},
        {ORC_RADIUS3D, ORC_ELEMENT, 4, 30, 16, 6, 5, 1, 2, 0, 0},
        {ORC_RADIUS3D, ORC_ELEMENT, 3, 12, 128, 3, 4, 0, 1, 0, 1},
        {ORC_SWA, ORC_ELEMENT, 7, 12, 16, 0, 0, 0, 0, 3, 0},
        {ORC_SWA, ORC_ELEMENT, 5, 30, 128, 0, 0, 0, 0, 2, 1},
        {ORC_DENSE, ORC_ELEMENT, 3, 17, 16, 0, 0, 0, 0, 0, 0},
    };
    char what[64];
    for (size_t i = 0; i < sizeof masks / sizeof masks[0]; ++i) {
        snprintf(what, sizeof what, "mask %zu (kind %d)", i, masks[i].kind);
        check_mask(&masks[i], what);
        check_attention(&masks[i], what);
    }
    check_eq4();
    check_salad();
    printf("oracle_check: %d checks passed\n", g_checks);
    return 0;
}

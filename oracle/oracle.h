/*
 * oracle.h -- plain fp64 CPU oracle for static sparse spatiotemporal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load liboracle.so.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * What it computes (sources are the pages on the method):
 *   - Radial Attention, section 2 eq. 2: softmax((Q K^T + M) / sqrt(d)) V with
 *     M in {-inf, 0}^{n x n}; an all-zero M is eq. 1 (standard attention).
 *   - Radial Attention, section 3 eq. 4: the 4-D radial mask over
 *     (query frame i, key frame j, query position k, key position l); the
 *     token index of (frame, position) is frame * s + position (section 1,
 *     the p_{js+l} index of eq. 3).
 *   - Token Radius Attention (both blog pages, "radius" design section): a
 *     token attends to the keys within temporal radius r_t and spatial radius
 *     r_s on the (t, h, w) token grid flattened t-h-w (3-D patch embedding
 *     section); keys outside the grid do not exist (no padding).
 *   - Vera 1.1 temporal module, section 2.1/2.2: frame-level causal sliding
 *     window, query frame i sees key frames [max(0, i - W + 1), i].
 *   - Radial Attention, section 6: sparsity is applied on 128 x 128 blocks; a
 *     block-granularity mask keeps a whole block iff any element is kept
 *     (ORC_BLOCK_ANY), or, as a second reading, iff eq. 4 holds for the block
 *     indices with block frames of s / block blocks (ORC_BLOCK_EQ4, radial
 *     only, s a multiple of the block edge).
 *   - Radial Attention, section 4 (complexity): the central-band term counts
 *     a "sink" beside the band.  sink_frames > 0 adds it in its plainest
 *     form: every query keeps every key of the first sink_frames frames.
 *   - SALAD, sections 2.1-2.2: the ReLU-kernel linear-attention branch over
 *     the same Q, K, V, its scalar gate (mean over tokens of a sigmoid of a
 *     linear map of the block input) and the gated, projected sum with the
 *     sparse branch.
 *
 * All mask arithmetic is integer.  Attention is fp64 over the exact input
 * values (bf16 or fp32, widened exactly).
 */
#ifndef TRA_ORACLE_H
#define TRA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_DENSE = 0, ORC_RADIAL = 1, ORC_RADIUS3D = 2, ORC_SWA = 3 };
enum { ORC_ELEMENT = 0, ORC_BLOCK_ANY = 1, ORC_BLOCK_EQ4 = 2 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };

typedef struct {
    int32_t kind;         /* ORC_* family                                    */
    int32_t granularity;  /* ORC_ELEMENT, ORC_BLOCK_ANY or ORC_BLOCK_EQ4     */
    int64_t f, s;         /* frames, tokens per frame; n = f * s             */
    int64_t block;        /* block edge for block granularity / counting     */
    int64_t grid_h, grid_w; /* RADIUS3D: s == grid_h * grid_w                */
    int64_t r_t, r_s;     /* RADIUS3D radii                                  */
    int64_t window;       /* SWA: frames seen, the current one included      */
    int64_t sink_frames;  /* keys of frames < sink_frames kept for all rows  */
} orc_mask;

/* Element predicate of the family (granularity ignored): 1 = kept (M = 0).
 * Includes the sink frames. */
int orc_keep(const orc_mask *m, int64_t q, int64_t t);

/* ORC_BLOCK_EQ4 block predicate: eq. 4 on (query block bq, key block bk)
 * with s / block blocks per frame, or bk inside the sink frames. */
int orc_keep_block_eq4(const orc_mask *m, int64_t bq, int64_t bk);

/* nb x nb kept-block matrix of the mask at its granularity (row = query
 * block): non-empty blocks for ORC_ELEMENT and ORC_BLOCK_ANY, the block
 * predicate for ORC_BLOCK_EQ4. */
void orc_block_keep(const orc_mask *m, uint8_t *out, int threads);

/* Dense n x n element matrix of the family's predicate (row = query). */
void orc_elem_matrix(const orc_mask *m, uint8_t *out);

/* Kept-element count of every (block-row, block-col) block of edge m->block
 * under the element predicate; blocks at the tail are cut at n.  Out holds
 * nb x nb int64 with nb = ceil(n / block).  Threads > 1 split block rows. */
void orc_block_counts(const orc_mask *m, int64_t *out, int threads);

/* Same as orc_block_counts for the listed block rows only: out holds
 * nrows x nb int64, row i = block row rows[i]. */
void orc_block_counts_rows(const orc_mask *m, const int64_t *rows, int64_t nrows, int64_t *out,
                           int threads);

/* Total kept elements of the element predicate. */
int64_t orc_kept_elements(const orc_mask *m, int threads);

/* Row-major 128-bit-per-row bitmap of one block (block edge m->block, which
 * must be 128 here): out[r * 4 + w] bit b = element (row qb*128 + r,
 * key kb*128 + w*32 + b) kept; elements beyond n read as 0. */
void orc_block_bits128(const orc_mask *m, int64_t qb, int64_t kb, uint32_t *out);

/* Number of keys each listed query row attends (same rule as
 * orc_attention_rows: element predicate, block_keep for ORC_BLOCK_ANY, the
 * block predicate for ORC_BLOCK_EQ4).  rows: nrows query indices. */
void orc_row_counts(const orc_mask *m, const uint8_t *block_keep, const int64_t *rows, int64_t nrows,
                    int64_t *out);

/* fp64 masked attention for a list of rows.
 *   q, k, v : [B, H, n, d] contiguous, dtype ORC_F32 (float) or ORC_BF16
 *             (raw bfloat16 bit patterns, uint16)
 *   mask    : the family; with ORC_BLOCK_ANY a key is kept iff its block
 *             is kept in block_keep (nb x nb bytes, row = query block), which
 *             the caller fills from orc_block_counts (> 0).  block_keep is
 *             ignored for ORC_ELEMENT and ORC_BLOCK_EQ4 (the latter tests
 *             orc_keep_block_eq4 for every key).
 *   scale   : multiplies Q K^T (1/sqrt(d) for eq. 1 and eq. 2)
 *   rows    : nrows triples (b, h, query index)
 *   o_out   : nrows x d; lse_out: nrows (natural log of the softmax
 *             denominator of the scaled scores).  A row with no kept key
 *             gets O = 0 and LSE = -inf.
 */
void orc_attention_rows(int dtype, const void *q, const void *k, const void *v,
                        int64_t B, int64_t H, int64_t n, int64_t d,
                        const orc_mask *mask, const uint8_t *block_keep,
                        double scale, const int64_t *rows, int64_t nrows,
                        double *o_out, double *lse_out, int threads);

/* fp64 gradients of eq. 2 for a list of rows (the backward pass of the
 * masked softmax attention).  With P the softmax of the scaled masked
 * scores, dO the gradient of the output and scale the score scale:
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(P o dP)),
 *   dQ = scale dS K,  dK = scale dS^T Q
 * Inputs as orc_attention_rows plus dO (same layout and dtype).
 *   q_rows : nq triples (b, h, query) whose dQ rows are returned in dq_out
 *            (nq x d)
 *   k_rows : nk triples (b, h, key) whose dK and dV rows are returned in
 *            dk_out, dv_out (nk x d)
 * A dK/dV row needs the softmax of every query that keeps the key, so its
 * cost is that of a full pass over the head. */
void orc_attention_bwd_rows(int dtype, const void *q, const void *k, const void *v, const void *dout,
                            int64_t B, int64_t H, int64_t n, int64_t d,
                            const orc_mask *mask, const uint8_t *block_keep, double scale,
                            const int64_t *q_rows, int64_t nq, double *dq_out,
                            const int64_t *k_rows, int64_t nk, double *dk_out, double *dv_out,
                            int threads);

/* SALAD linear branch (page "SALAD", section 2.1): ReLU-kernel linear
 * attention over the same Q, K, V, for a list of rows.  With phi = ReLU and
 * w_t = phi(Q[q]) . phi(K[t]) over every key t of the (b, h):
 *   O[q] = sum_t w_t V[t] / (sum_t w_t + eps)
 * (the attention form; a linear-time kernel evaluates it as
 * phi(Q) (phi(K)^T V) / (phi(Q) . sum_t phi(K[t]) + eps)).
 * Layout and dtypes as orc_attention_rows. */
void orc_linear_attention_rows(int dtype, const void *q, const void *k, const void *v, int64_t B, int64_t H,
                               int64_t n, int64_t d, double eps, const int64_t *rows, int64_t nrows,
                               double *o_out, int threads);

/* SALAD gate (page "SALAD", section 2.2): a learned linear map of the block
 * input to one value per token, a sigmoid, then the mean over the sequence,
 * one scalar per sample:
 *   g[b] = (1 / N) sum_n sigmoid(x[b, n, :] . w + bias),
 *   sigmoid(z) = 1 / (1 + exp(-z)).
 *   x : [B, N, C] contiguous (dtype), w : [C] (dtype), g_out : B doubles. */
void orc_salad_gate(int dtype, const void *x, const void *w, double bias, int64_t B, int64_t N, int64_t C,
                    double *g_out, int threads);

/* SALAD output (page "SALAD", sections 2.1-2.2): the sparse branch plus the
 * gated projection of the linear branch, in the merged-head channel space
 * c = h * d + e (C = H * d channels):
 *   out[b, n, c'] = O_s[b, n, c'] + g[b] * (sum_c O_l[b, n, c] W[c', c] + bias[c'])
 * O_s, O_l : [B, H, N, d] contiguous (dtype), so channel c of token n is
 *            element [b, c / d, n, c % d];
 * W        : [C, C] row-major (dtype), the projection (out = in W^T);
 * bias     : C doubles, or NULL for none;  g : B doubles;
 * rows     : nrows pairs (b, n);  out : nrows x C. */
void orc_salad_output_rows(int dtype, const void *o_sparse, const void *o_lin, const void *w, const double *bias,
                           const double *g, int64_t B, int64_t H, int64_t N, int64_t d, const int64_t *rows,
                           int64_t nrows, double *out, int threads);

#ifdef __cplusplus
}
#endif
#endif

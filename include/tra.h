/*
 * tra.h -- C ABI of the static sparse spatiotemporal attention library
 * (libtra.so), built for AMD Instinct MI355X (gfx950).
 *
 * The library computes masked attention over video tokens,
 *
 *     O = softmax((Q K^T + M) * scale) V,   M in {-inf, 0}^{n x n},
 *
 * Radial Attention (NeurIPS 2025) section 2, eq. 2 (eq. 1 when M = 0), with
 * the scale 1/sqrt(d) of those equations unless the caller passes another.
 * M is static: it depends only on the frame count f, the tokens per frame s
 * and the family parameters, never on Q, K, V.  The families:
 *
 *   TRA_MASK_RADIAL      Radial Attention section 3, eq. 4.  Token index =
 *                        frame * s + position.  Query (frame i, position k)
 *                        keeps key (frame j, position l) iff, with
 *                        r = floor(log2(max(|i-j|, 1))):
 *                          2^r <= s and |k-l| + 1 <= s / 2^r, or
 *                          |i-j| mod ceil(2^r / s) == 0 and k == l.
 *   TRA_MASK_RADIUS3D    Token Radius Attention (radius design section of
 *                        both blog pages): tokens on a (f, grid_h, grid_w)
 *                        grid flattened t-h-w; keep iff |dt| <= r_t and
 *                        max(|dh|, |dw|) <= r_s.  Keys off the grid do not
 *                        exist (no padding).
 *   TRA_MASK_SWA_CAUSAL  Vera 1.1 temporal module, sections 2.1-2.2:
 *                        query frame i keeps every token of key frames
 *                        max(0, i - window + 1) .. i.
 *   TRA_MASK_DENSE       every entry kept (eq. 1).
 *
 * Any family may add sink frames: every query also keeps every key of the
 * first sink_frames frames (the "sink" beside the central band in Radial
 * Attention section 4's count; the pages give no other form of it).
 *
 * Radial Attention section 6 applies sparsity on 128 x 128 blocks; the mask
 * is compiled once into a block bitmap, a per-query-block CSR list of kept
 * key blocks and 128 x 128 element bitmasks for the kept blocks that are only
 * partly kept.  TRA_GRAN_BLOCK_ANY keeps a whole block iff any element in it
 * is kept.  TRA_GRAN_BLOCK_EQ4 (radial only) reads the block sparsity as eq. 4
 * applied to the block indices, with s / 128 blocks per frame: a block is
 * kept or dropped whole by the same rule that keeps a token pair (sink frames
 * keep whole block columns).
 *
 * Conventions for every call:
 *   - Return TRA_OK (0) or a negative tra_status.  Argument, shape, dtype and
 *     stride errors are detected on the host before anything is enqueued.
 *   - Device work is asynchronous on the caller's HIP stream (NULL = the
 *     default stream); faults inside kernels surface at the caller's next
 *     synchronisation.  TRA_ERR_HIP means a HIP runtime call failed; its
 *     hipError_t is kept in tra_last_hip_error() (per thread).
 *   - Device pointers are HIP device (or managed) memory of the current
 *     device.  No call keeps a pointer to caller memory after it returns.
 */
#ifndef TRA_H
#define TRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRA_OK = 0,
    TRA_ERR_INVALID = -1,     /* null pointer, value out of range           */
    TRA_ERR_UNSUPPORTED = -2, /* valid request the library does not handle */
    TRA_ERR_SHAPE = -3,       /* tensor shapes disagree with each other/mask */
    TRA_ERR_OOM = -4,         /* device allocation failed                   */
    TRA_ERR_HIP = -5          /* other HIP runtime failure                  */
} tra_status;

typedef enum {
    TRA_MASK_DENSE = 0,
    TRA_MASK_RADIAL = 1,
    TRA_MASK_RADIUS3D = 2,
    TRA_MASK_SWA_CAUSAL = 3
} tra_mask_kind;

typedef enum {
    TRA_GRAN_ELEMENT = 0,   /* exact element mask; partial blocks carry bits */
    TRA_GRAN_BLOCK_ANY = 1, /* 128 x 128 block kept iff any element kept     */
    TRA_GRAN_BLOCK_EQ4 = 2  /* eq. 4 on block indices (radial, s % 128 == 0) */
} tra_granularity;

typedef enum { TRA_F32 = 0, TRA_BF16 = 1 } tra_dtype;

/* Family parameters.  Fields a family does not use must be 0.
 *   granularity  tra_granularity
 *   block        block edge; must be 0 (= 128) or 128
 *   grid_h/w     RADIUS3D: s == grid_h * grid_w, grid_h, grid_w >= 1
 *   r_t, r_s     RADIUS3D radii, >= 0
 *   window       SWA_CAUSAL: frames seen including the current one, >= 1
 *   sink_frames  any family: leading key frames kept for every query, >= 0
 *                (values above f act as f)
 *   reserved     must be 0                                                  */
typedef struct {
    int32_t granularity;
    int32_t block;
    int32_t grid_h, grid_w;
    int32_t r_t, r_s;
    int32_t window;
    int32_t sink_frames;
    int32_t reserved[8];
} tra_mask_params;

typedef struct tra_mask tra_mask; /* opaque; owns its device buffers */

typedef struct {
    int64_t n;              /* tokens = f * s                               */
    int64_t f, s;
    int64_t nqb, nkb;       /* query / key blocks = ceil(n / 128)           */
    int64_t kept_blocks;    /* CSR entries (non-empty blocks)               */
    int64_t partial_blocks; /* kept blocks that carry an element bitmask    */
    int64_t kept_elems;     /* (q, t) pairs, q, t < n, attended per (b, h)  */
    int64_t pred_elems;     /* pairs kept by the family's element predicate
                               (with sink frames; eq. 4 on tokens also for
                               TRA_GRAN_BLOCK_EQ4)                           */
    int64_t min_row_blocks, max_row_blocks;
    int64_t bitmap_words;   /* uint32 words per bitmap row = ceil(nkb / 32) */
    int64_t work_items;     /* bf16 kernel work items per (b, h): query blocks
                               paired by key-block overlap, plus singles     */
    int64_t tile_loads;     /* K/V tiles the bf16 kernel loads per (b, h)    */
    int32_t kind, granularity;
    int64_t bwd_work_items; /* backward dK/dV work items per (b, h): key
                               blocks paired by query-block overlap          */
    int64_t bwd_tile_loads; /* Q/dO tiles the dK/dV kernel loads per (b, h)  */
} tra_mask_info;

/* A [B, H, N, D] tensor view.  stride[] in elements, order B, H, N, D;
 * stride[3] must be 1; stride[2] (row pitch) a multiple of 8 elements and
 * data 16-byte aligned. */
typedef struct {
    void *data;
    int32_t dtype; /* tra_dtype */
    int32_t reserved;
    int64_t B, H, N, D;
    int64_t stride[4];
} tra_tensor;

/*
 * tra_build_mask -- compile the static mask for n = f * s tokens.
 *
 * Defines M of eq. 2 from the family (see the list at the top of this file)
 * and stores it at 128 x 128 block granularity (Radial Attention section 6).
 * f >= 1, s >= 1, n < 2^31.  n need not be a multiple of 128: the last
 * block row/column is cut at n and every kept block that reaches past n
 * carries an element bitmask that drops the missing keys.
 *
 * Runs the mask-builder kernels on `hip_stream` and waits for them (the mask build
 * is synchronous; it is meant to run once per (f, s, kind, params)).  On
 * success *out owns device memory until tra_mask_free.  On failure *out is
 * NULL.  Errors: TRA_ERR_INVALID (null out/params, f or s < 1, unknown kind
 * or granularity, negative radius or sink_frames, window < 1, nonzero unused
 * field, TRA_GRAN_BLOCK_EQ4 with a kind other than RADIAL),
 * TRA_ERR_UNSUPPORTED (block not 0/128, n >= 2^31, TRA_GRAN_BLOCK_EQ4 with
 * s not a multiple of 128), TRA_ERR_SHAPE (RADIUS3D with
 * s != grid_h * grid_w), TRA_ERR_OOM, TRA_ERR_HIP.
 */
tra_status tra_build_mask(int64_t f, int64_t s, int32_t kind, const tra_mask_params *params,
                          void *hip_stream, tra_mask **out);

/*
 * tra_sparse_attn_fwd -- O = softmax((Q K^T + M) * scale) V  (eq. 2).
 *
 * Q, K, V, O: [B, H, N, D] views, one dtype for all four (TRA_BF16: bf16
 * inputs taken as given, fp32 accumulation of the scores, exponentials and
 * sums, the probabilities rounded to bf16 for the P V product, O rounded to
 * nearest-even bf16; TRA_F32: fp32 throughout).  N == mask n; D in
 * {64, 128}.  O must not overlap Q, K or V.
 * LSE: NULL or device float[B * H * N] (contiguous [B, H, N]) receiving the
 * natural log of each row's softmax denominator, ln sum_t exp(scale * q.k_t)
 * over kept keys.  scale <= 0 selects 1/sqrt(D).  Rows whose every key is
 * masked (impossible for the families above) get O = 0 and LSE = -inf.
 *
 * The mask is shared by every (b, h).  Asynchronous on hip_stream; allocates
 * nothing.  The mask holds the work-queue counters of the kernel and, for
 * launches with few work items per compute unit, the records through which
 * the two halves of an item split over its key blocks are combined (in a
 * fixed order: results are the same bit for bit on every call).  Calls that
 * use the same mask must therefore not run concurrently (same stream is
 * fine).
 * B == 0 or H == 0 returns TRA_OK without launching.
 * Errors: TRA_ERR_INVALID (null tensor/mask/data), TRA_ERR_SHAPE (shapes
 * disagree or N != n), TRA_ERR_UNSUPPORTED (D not 64/128, mixed dtypes,
 * bad stride or alignment, more than 2^31 work items), TRA_ERR_HIP.
 */
tra_status tra_sparse_attn_fwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V,
                               const tra_mask *mask, tra_tensor *O, float *LSE, float scale,
                               void *hip_stream);

/*
 * tra_sparse_attn_bwd_workspace_bytes -- device workspace bytes that
 * tra_sparse_attn_bwd needs for B x H heads of N rows of width D: two fp32
 * values per row, each array 256-byte aligned (about 8 B H N bytes).
 * Returns 0 for negative sizes or D not 64/128.
 */
size_t tra_sparse_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);

/*
 * tra_sparse_attn_bwd -- gradients of eq. 2 (the backward pass of
 * tra_sparse_attn_fwd with the same mask and scale).
 *
 * With P the forward's probabilities (recomputed from Q, K and the saved
 * LSE), dO the gradient of O and delta = rowsum(dO o O):
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),
 *   dK = scale dS^T Q,  dQ = scale dS K.
 * P is recomputed from the raw dot products q.k in fp32 as
 * exp(scale q.k - LSE), so that its rows sum to 1 against the saved LSE.
 * Q, K, V, O, dO, dQ, dK, dV: [B, H, N, D] views of one dtype (same rules
 * as the forward).  TRA_BF16: MFMA products of bf16 operands (P and dS
 * rounded to bf16), fp32 accumulation, gradients rounded to bf16.  TRA_F32:
 * fp32 arithmetic throughout (vector ALU; meant for the small fp32
 * workloads).
 * O and LSE must be the forward outputs for these Q, K, V, mask and scale.
 * workspace: device memory of at least tra_sparse_attn_bwd_workspace_bytes
 * bytes, 256-byte aligned, owned by the caller; overwritten (it holds delta
 * and -LSE log2(e) per row while the call runs).
 * The outputs must not overlap the inputs, the workspace or each other.
 * Asynchronous; allocates nothing; the same mask must not be used by a
 * concurrent call.  Results are deterministic (no atomics).  B == 0 or
 * H == 0 returns TRA_OK.
 * Errors: TRA_ERR_INVALID (null tensor/mask/data/LSE/workspace, workspace
 * too small or misaligned), TRA_ERR_SHAPE, TRA_ERR_UNSUPPORTED (mixed
 * dtypes, D not 64/128, bad stride or alignment), TRA_ERR_HIP.
 */
tra_status tra_sparse_attn_bwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V,
                               const tra_tensor *O, const tra_tensor *dO, const float *LSE,
                               const tra_mask *mask, tra_tensor *dQ, tra_tensor *dK, tra_tensor *dV,
                               void *workspace, size_t workspace_bytes, float scale, void *hip_stream);

/*
 * Frame-streaming K/V cache for the frame sliding-window causal family (Vera
 * 1.1 temporal module, section 3.1): keeps the keys and values of the last
 * `window` frames in a ring; appending a frame evicts the oldest one once the
 * ring is full.  tra_kvcache_attn then computes the rows of the newest frame
 * of TRA_MASK_SWA_CAUSAL attention (query frame i over key frames
 * max(0, i - window + 1) .. i) without the earlier frames' queries.
 *
 * tra_kvcache_create -- allocate the ring (2 x B x H x window x s x D bf16)
 *   and a split workspace for B heads-batch, H heads, s tokens per frame
 *   (a multiple of 128), head dim D in {64, 128}, dtype TRA_BF16.  Errors:
 *   TRA_ERR_INVALID (null out, a size < 1), TRA_ERR_UNSUPPORTED (other dtype,
 *   D, or s % 128 != 0), TRA_ERR_OOM, TRA_ERR_HIP.
 * tra_kvcache_append -- copy K, V of the next frame ([B, H, s, D] views,
 *   same rules as the attention tensors) into the ring (asynchronous on the
 *   stream; the frame counter advances on the host).
 * tra_kvcache_attn -- O = softmax(Q K^T * scale) V for Q, O [B, H, s, D] of
 *   the newest frame over every cached frame; LSE as tra_sparse_attn_fwd (NULL
 *   skips it).  The keys are split over workgroups and the partial results
 *   merged (asynchronous; allocates nothing).  TRA_ERR_INVALID when nothing
 *   has been appended.
 * tra_kvcache_get_frames -- frames appended since creation/reset and frames
 *   currently cached (<= window).
 * tra_kvcache_reset -- start a new sequence (no device work).
 * tra_kvcache_free -- release the cache (NULL is ignored); the caller makes
 *   sure no call using it is still queued.
 * Calls on one cache must not run concurrently.
 */
typedef struct tra_kvcache tra_kvcache;
tra_status tra_kvcache_create(int64_t B, int64_t H, int64_t s, int64_t D, int32_t window, int32_t dtype,
                              tra_kvcache **out);
tra_status tra_kvcache_append(tra_kvcache *cache, const tra_tensor *K, const tra_tensor *V, void *hip_stream);
tra_status tra_kvcache_attn(tra_kvcache *cache, const tra_tensor *Q, tra_tensor *O, float *LSE, float scale,
                            void *hip_stream);
tra_status tra_kvcache_get_frames(const tra_kvcache *cache, int64_t *appended, int64_t *cached);
tra_status tra_kvcache_reset(tra_kvcache *cache);
void tra_kvcache_free(tra_kvcache *cache);

/*
 * SALAD linear branch (page "SALAD", section 2.1): ReLU-kernel linear
 * attention over the same Q, K, V as the sparse branch, for every row of
 * every (b, h):
 *     O[q] = phi(Q[q]) (sum_t phi(K[t])^T V[t]) / (phi(Q[q]) . sum_t phi(K[t]) + eps),
 * phi = ReLU, O(N D^2) work.  The gate and the output projection of the
 * branch are trained layers of the model around this call.
 *
 * tra_linear_attn_workspace_bytes -- bytes of device workspace the call
 *   needs for [B, H, N, D] (0 for an unsupported D).
 * tra_linear_attn_fwd -- Q, K, V, O: [B, H, N, D] bf16 views (forward's
 *   rules; any N >= 1), eps >= 0 (1e-6 is typical), workspace: device
 *   memory of at least that many bytes, 256-byte aligned, owned by the
 *   caller and overwritten.  Accumulation in fp32; the d x d summary is
 *   applied as a pair of bf16 values (about 16 significant bits); O rounded
 *   to bf16.  Asynchronous; allocates nothing.  Errors: TRA_ERR_INVALID
 *   (null tensor/data/workspace, workspace too small or misaligned,
 *   eps < 0), TRA_ERR_SHAPE, TRA_ERR_UNSUPPORTED (dtype, D, stride or
 *   alignment), TRA_ERR_HIP.
 */
size_t tra_linear_attn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);
tra_status tra_linear_attn_fwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V, tra_tensor *O,
                               float eps, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * SALAD gate and output (page "SALAD", section 2.2 for the gate; section 2.1
 * for the one projection layer the linear branch adds).  The gate scales the
 * linear branch by one scalar per sample:
 *     g[b] = (1 / N) sum_n sigmoid(X[b, n, :] . w + bias),
 * the mean over the tokens of a sigmoid of a learned linear map of the
 * block input X.  The branch output is then projected and added to the
 * sparse branch in the merged-head channel space c = h * D + e (C = H * D
 * channels; channel c of token n is element [b, c / D, n, c % D] of a
 * [B, H, N, D] tensor):
 *     out[b, n, c'] = O_sparse[b, n, c'] + g[b] * (sum_c O_lin[b, n, c] W[c', c] + bias[c']).
 * The weights are the model's (trained) parameters; the library only
 * applies them.  A caller that drops the linear branch when g is small
 * reads g back before deciding to call tra_salad_combine.
 *
 * tra_salad_gate_workspace_bytes -- device workspace bytes tra_salad_gate
 *   needs for B samples of N tokens (256-byte multiple).
 * tra_salad_gate -- X: the block input as a [B, 1, N, C] bf16 view (H = 1,
 *   D = C channels, C a multiple of 8 and at most 8192; unit channel
 *   stride; B and N strides multiples of 8 elements; 16-byte aligned);
 *   w: device bf16 [C], 16-byte aligned; bias: the map's scalar bias;
 *   gate: device fp32 [B], written; workspace: device memory of at least
 *   that many bytes, 256-byte aligned, owned by the caller and overwritten.
 *   fp32 sums in a fixed order (bitwise reproducible).  Asynchronous;
 *   allocates nothing.  Errors: TRA_ERR_INVALID (null pointer, workspace too
 *   small or misaligned, N = 0 with B > 0), TRA_ERR_SHAPE (negative sizes,
 *   H != 1), TRA_ERR_UNSUPPORTED (dtype, C, strides, alignment),
 *   TRA_ERR_HIP.
 * tra_salad_combine -- O_sparse, O_lin, out: [B, H, N, D] bf16 views of one
 *   shape (forward's stride rules, D = 64 or 128, C = H * D a multiple of
 *   64); W: device bf16 [C][C] row-major (row c' holds the weights of output
 *   channel c', as a PyTorch Linear weight), 16-byte aligned; bias: device
 *   fp32 [C], 16-byte aligned, or NULL for none; gate: device fp32 [B] (for
 *   example from tra_salad_gate).  out may be O_sparse itself (same data
 *   and strides: every element is read before the same thread writes it),
 *   never O_lin.  fp32 accumulation; out rounded to bf16.  Asynchronous;
 *   allocates nothing.  Errors: TRA_ERR_INVALID (null pointer, out sharing
 *   O_lin's data), TRA_ERR_SHAPE, TRA_ERR_UNSUPPORTED (dtype, D, C, strides,
 *   alignment, sizes past 2^31 tokens), TRA_ERR_HIP.
 */
size_t tra_salad_gate_workspace_bytes(int64_t B, int64_t N);
tra_status tra_salad_gate(const tra_tensor *X, const void *w, float bias, float *gate, void *workspace,
                          size_t workspace_bytes, void *hip_stream);

/*
 * tra_salad_gate_noalloc -- tra_salad_gate for callers that cannot allocate
 * device memory or bring a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (minus the
 * workspace), checks, kernels and results (bit for bit) as tra_salad_gate;
 * the partial sums go to a fixed array in the library's device memory
 * (256 KB, 65536 floats, one copy per device, held until the process ends).
 * Calls no allocating routine.  Limit: B * min(1024, ceil(N / 64)) <= 65536
 * (any N when B <= 64); larger requests return TRA_ERR_UNSUPPORTED before
 * anything is enqueued.  Every call on a device shares that array, so calls
 * that overlap in time on one device (two streams, two threads) race; calls
 * ordered on one stream are safe.  Errors: as tra_salad_gate (no workspace
 * errors), TRA_ERR_UNSUPPORTED past the limit, TRA_ERR_HIP.
 */
tra_status tra_salad_gate_noalloc(const tra_tensor *X, const void *w, float bias, float *gate, void *hip_stream);
tra_status tra_salad_combine(const tra_tensor *O_sparse, const tra_tensor *O_lin, const void *W, const float *bias,
                             const float *gate, tra_tensor *out, void *hip_stream);

/* Copy the host-side summary filled at build time.  No device work. */
tra_status tra_mask_get_info(const tra_mask *mask, tra_mask_info *out);

/*
 * tra_mask_export -- copy the compiled mask to host buffers (synchronous).
 * Any pointer may be NULL to skip that part.  Sizes from tra_mask_info:
 *   bitmap    uint32[nqb * bitmap_words]; bit (kb % 32) of word
 *             [qb * bitmap_words + kb / 32] = block (qb, kb) kept
 *   row_ptr   int32[nqb + 1]; CSR offsets of each query block's kept blocks
 *   col_idx   int32[kept_blocks]; kept key blocks, ascending within a row
 *   emask_idx int32[kept_blocks]; -1 = whole block kept, else the index of
 *             its bitmask (partial blocks numbered in CSR order)
 *   emask     uint32[partial_blocks * 128 * 4]; row r of a partial block is
 *             4 words, bit b of word w = key (w * 32 + b) of the block kept
 *   order     int32[nqb]; the query blocks in chunks of 64 consecutive
 *             blocks, each chunk ordered by decreasing kept-block count
 *             (ties by index): the order in which the attention kernels
 *             take the blocks of one chunk
 */
tra_status tra_mask_export(const tra_mask *mask, uint32_t *bitmap, int32_t *row_ptr,
                           int32_t *col_idx, int32_t *emask_idx, uint32_t *emask, int32_t *order);

/* Release the mask's device memory.  NULL is ignored.  The caller makes sure
 * no kernel that uses the mask is still queued. */
void tra_mask_free(tra_mask *mask);

/* Static, never-NULL name of a status code. */
const char *tra_status_string(tra_status s);

/* hipError_t of the last TRA_ERR_HIP / TRA_ERR_OOM returned on this thread
 * (0 if none). */
int32_t tra_last_hip_error(void);

/* Library version as 10000 * major + 100 * minor + patch. */
int32_t tra_version(void);

/*
 * tra_probe_mfma_peak -- a measurement helper, not part of the attention
 * path: `blocks` workgroups of 8 waves (two per SIMD) each run `iterations`
 * rounds of 4 independent v_mfma_f32_32x32x16_bf16 on register operands, with
 * no memory traffic in the loop; one float per workgroup is written to
 * `out` (device float[blocks]) so that the loop is kept.  The caller times
 * the launch on `hip_stream`; *flops receives the MFMA flops it executes
 * (blocks x 8 x 4 x iterations x 32768).  With one workgroup per compute
 * unit this gives the bf16 MFMA rate the chip sustains under full MFMA load,
 * the measured peak beside the data-sheet one.  Asynchronous; allocates
 * nothing.  Errors: TRA_ERR_INVALID (iterations < 1, blocks < 1, null out
 * or flops), TRA_ERR_HIP.
 */
tra_status tra_probe_mfma_peak(int64_t iterations, int32_t blocks, float *out, int64_t *flops, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* TRA_H */

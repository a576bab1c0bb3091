// Internal declarations shared by the HIP sources of libtra.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tra.h"
#include "tra_sched.h"

namespace tra {

// Per-XCD work queues (chunks of kChunk query blocks or kPairChunk pairs,
// see tra_sched.h): the queue buffer holds kQueues counters and one
// finished-workgroup counter.
constexpr int kQueues = 8;
constexpr int kQueueWords = 16;
// Split items of the forward's tail mode (see WorkQueue): at most one per
// slot of a queue's last chunk.  Each half leaves its partial state
// (unnormalised O^T fragments, row maximum and lane sums, in each lane's
// register order) in a record of its own, 2 x split + half, which the half
// that finishes second reads.
constexpr int kSplitSlots = kQueues * kPairChunk;
constexpr int kSplitLaneFloats = 128 / 32 * 16 + 2;          // O^T fragments at D = 128, m, l
constexpr int64_t kSplitRecFloats = 8 * 64 * kSplitLaneFloats;  // 8 waves x 64 lanes

// Mask family as seen by device code.
struct MaskDesc {
    int32_t kind;
    int32_t granularity;
    int32_t n, f, s;
    int32_t grid_h, grid_w, r_t, r_s, window;
    int32_t sink_frames;
};

// Block class written by the classifier.
enum : uint8_t { kEmpty = 0, kFull = 1, kPartial = 2 };

// Device view of a compiled mask, passed to the attention kernels by value.
//
// Besides the per-query-block CSR, the builder pairs query blocks whose kept
// key blocks largely coincide (greedy, by Jaccard overlap) and stores, per
// pair, the sorted union of their key blocks with one emask index per member
// (-1 full, >= 0 bitmask, kAbsent not kept).  A kernel that serves both
// members of a pair from one K/V tile halves the tile traffic.
struct MaskDev {
    const int32_t *row_ptr;    // [nqb + 1]
    const int32_t *col_idx;    // [nnz]
    const int32_t *emask_idx;  // [nnz], -1 = full block
    const uint32_t *emask;     // [npartial][128][4]
    const int32_t *order;      // [nqb] chunk-wise heaviest-first query blocks
    const int32_t *pair_rows;  // [npairs][2] query blocks (second = -1: unpaired)
    const int32_t *pair_ptr;   // [npairs + 1] offsets into the union schedule
    const int32_t *u_col;      // [nunion] key block
    const int32_t *u_em;       // [nunion][2] emask index per member
    const int32_t *pair_order; // [npairs] chunk-wise heaviest-first pairs
    uint32_t *queue;           // [kQueueWords] XCD queue counters, finished-group counter
    uint32_t *split_ctr;       // [kSplitSlots] halves of a split item done (reset by the second)
    float *split_ws;           // [2 * kSplitSlots][kSplitRecFloats] partial state of each half
    int32_t nqb;
    int32_t npairs;
    // The same schedule over key blocks (columns of the block mask), for the
    // kernels that accumulate per key block: pairs of key blocks whose query
    // blocks largely coincide, and the merged query-block list of each pair
    // with the emask index of block (query block, member key block).
    const int32_t *t_pair_cols;   // [t_npairs][2] key blocks (second = -1: unpaired)
    const int32_t *t_pair_ptr;    // [t_npairs + 1]
    const int32_t *t_u_row;       // [t_nunion] query block
    const int32_t *t_u_em;        // [t_nunion][2]
    const int32_t *t_pair_order;  // [t_npairs]
    int32_t t_npairs;
};

}  // namespace tra

struct tra_mask {
    tra_mask_info info;
    tra::MaskDesc desc;
    int device;
    // device buffers (owned)
    uint32_t *bitmap;
    int32_t *row_ptr;
    int32_t *col_idx;
    int32_t *emask_idx;
    uint32_t *emask;
    int32_t *order;
    int32_t *pair_rows;
    int32_t *pair_ptr;
    int32_t *u_col;
    int32_t *u_em;
    int32_t *pair_order;
    int32_t npairs;
    int32_t max_pair_tiles;  // longest item of the pair schedule (key blocks)
    uint32_t *queue;
    uint32_t *split_ctr;
    float *split_ws;
    int32_t *t_pair_cols;
    int32_t *t_pair_ptr;
    int32_t *t_u_row;
    int32_t *t_u_em;
    int32_t *t_pair_order;
    int32_t t_npairs;
    int64_t t_nunion;
};

namespace tra {

// Workgroups of `kern` (launched with `threads` threads and no dynamic LDS)
// that the current device holds at once: compute units times resident
// workgroups per unit (at least one per unit).  Queried from the runtime once
// per (device, kernel) and kept for the life of the process, so that a launch
// costs no device queries.
hipError_t resident_workgroups(const void *kern, int threads, long long *out);

// Mask builder (mask_build.hip).  All enqueue on `st`.
hipError_t launch_classify(const MaskDesc &m, int nqb, int nkb, uint8_t *cls, int32_t *cnt,
                           hipStream_t st);
hipError_t launch_row_stats(const MaskDesc &m, int nqb, int nkb, const uint8_t *cls,
                            const int32_t *cnt, int32_t *row_blocks, int32_t *row_partial,
                            long long *row_pred, long long *row_eff, hipStream_t st);
hipError_t launch_compact(int nqb, int nkb, const uint8_t *cls, const int32_t *row_ptr,
                          const int32_t *part_ptr, int32_t *col_idx, int32_t *emask_idx,
                          int32_t *part_list, hipStream_t st);
hipError_t launch_fill_emask(const MaskDesc &m, int npartial, const int32_t *part_list, int nkb,
                             uint32_t *emask, hipStream_t st);
hipError_t launch_bitmap(int nqb, int nkb, int words, const uint8_t *cls, uint32_t *bitmap,
                         hipStream_t st);

// Attention forward (attn_fwd.hip).
struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t sq[3], sk[3], sv[3], so[3];  // strides (elements) of B, H, N
    int32_t B, H, N, D;
    float scale_log2;  // scale * log2(e)
    MaskDev mask;
    // Key rows (copies past Nk repeat row Nk - 1); N for the masked call.
    int32_t Nk;
    // Split-key mode (frame streaming over a K/V ring): query blocks are
    // paired in order, every key block in [0, nkv_tiles) is kept whole, and
    // split x of the key blocks writes its normalised partial output and
    // log2-sum-exp to part_o / part_lse, merged by a second kernel.
    float *part_o;     // [nsplit][B * H * N][D]
    float *part_lse;   // [nsplit][B * H * N]
    int32_t nsplit, split_tiles, nkv_tiles, stream_pairs;
    // Tail mode of the masked call (see WorkQueue): items of the queues'
    // last chunks with at least split_min key blocks run as two halves.
    int32_t tail_split, split_min;
    int32_t max_pair_tiles;  // longest item of the pair schedule (key blocks)
};
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st);
// Split-key launch (see AttnArgs) followed by the merge into a.o / a.lse.
hipError_t launch_attn_stream_bf16(const AttnArgs &a, hipStream_t st);
// Copy two [B, H, rows, D] bf16 views (K and V) into rows row0 .. of their
// contiguous [B, H, ring_rows, D] buffers, in one launch.
hipError_t launch_ring_copy(const void *k_src, const int64_t *s_k, void *ring_k, const void *v_src,
                            const int64_t *s_v, void *ring_v, int64_t B, int64_t H, int64_t rows, int64_t D,
                            int64_t ring_rows, int64_t row0, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st);

// Attention backward (attn_bwd_bf16.hip): gradients of eq. 2 from the saved
// LSE.  delta[row] = dO[row] . O[row] is computed first into a caller buffer.
struct BwdArgs {
    AttnArgs f;          // q, k, v, strides, shape, scale, mask (o unused)
    const void *o, *dout;
    void *dq, *dk, *dv;
    const float *lse;
    // workspace: delta = rowsum(dO o O) and nlse = -LSE log2(e), fp32 per row
    float *delta, *nlse;
    int64_t s_o[3], s_do[3], s_dq[3], s_dk[3], s_dv[3];
};
// Byte offsets of the backward workspace's parts (256-byte aligned) and its size.
struct BwdWorkspace {
    size_t delta, nlse, bytes;
};
BwdWorkspace bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t D);
hipError_t launch_attn_bwd_bf16(const BwdArgs &a, hipStream_t st);
// fp32 inputs (attn_bwd_f32.hip): the same gradients in fp32 arithmetic.
hipError_t launch_attn_bwd_f32(const BwdArgs &a, hipStream_t st);

// SALAD linear branch (attn_linear_bf16.hip).
size_t linear_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);
hipError_t launch_linear_attn_bf16(const void *q, const int64_t *sq, const void *k, const int64_t *sk,
                                   const void *v, const int64_t *sv, void *o, const int64_t *so, int64_t B,
                                   int64_t H, int64_t N, int64_t D, float eps, void *ws, hipStream_t st);

}  // namespace tra

// Internal declarations shared by the HIP sources of libtra.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tra.h"

namespace tra {

constexpr int kBlock = 128;  // mask block edge (Radial Attention section 6)

// Mask family as seen by device code.
struct MaskDesc {
    int32_t kind;
    int32_t granularity;
    int32_t n, f, s;
    int32_t grid_h, grid_w, r_t, r_s, window;
};

// Block class written by the classifier.
enum : uint8_t { kEmpty = 0, kFull = 1, kPartial = 2 };

// Device view of a compiled mask, passed to the attention kernels by value.
struct MaskDev {
    const int32_t *row_ptr;    // [nqb + 1]
    const int32_t *col_idx;    // [nnz]
    const int32_t *emask_idx;  // [nnz], -1 = full block
    const uint32_t *emask;     // [npartial][128][4]
    const int32_t *order;      // [nqb] query blocks, heaviest first
    uint32_t *queue;           // [2] work-queue counter, finished-group counter
    int32_t nqb;
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
    uint32_t *queue;
};

namespace tra {

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
};
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st);

}  // namespace tra

// Helpers shared by the attention kernels.
#pragma once

#include "tra_internal.h"

namespace tra {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;

// {r[0], r[1]} = {v[lane], v[lane ^ 32]} in some order on every lane, so a
// symmetric combine of the two gives the same bits on both partner lanes.
__device__ inline float lane_pair_max(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float lane_pair_sum(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// XCD-affine work queues.  The work items of one (batch, head) -- query
// blocks, or pairs of them -- are taken in chunks of `chunk` consecutive
// items; chunk g of the (batch * head)-major chunk list belongs to the queue
// of XCD g % kQueues, so the workgroups resident on one XCD (sharing its L2)
// work on neighbouring query blocks, whose kept key blocks largely coincide.
// A workgroup drains its own XCD's queue first and then steals from the
// others.  Slot k of queue x is slot k % chunk of chunk x + kQueues *
// (k / chunk); slots past the last item of a (batch, head) are skipped, and
// `order` permutes the items inside each chunk.
struct WorkQueue {
    uint32_t *ctr;
    const __attribute__((address_space(4))) int32_t *order;
    int per_bh, chunk, nch, total_chunks;

    __device__ WorkQueue(uint32_t *queue, const int32_t *order_, int per_bh_, int chunk_, int bh_count)
        : ctr(queue), order((const __attribute__((address_space(4))) int32_t *)order_), per_bh(per_bh_),
          chunk(chunk_), nch((per_bh_ + chunk_ - 1) / chunk_), total_chunks(bh_count * nch)
    {
    }

    // Next item of the workgroup (wave-uniform results); false when every
    // queue is drained.  `x` is the queue being drained (start: this XCD),
    // `tries` how many queues have been left behind.
    __device__ bool next(int &x, int &tries, int *slot, int &bh, int &item)
    {
        for (;;) {
            if (tries >= kQueues)
                return false;
            const int chunks_x = total_chunks > x ? (total_chunks - x + kQueues - 1) / kQueues : 0;
            const long long len = (long long)chunks_x * chunk;
            if (threadIdx.x == 0)
                *slot = (int)atomicAdd(&ctr[x], 1u);
            __syncthreads();
            const int k = __builtin_amdgcn_readfirstlane(*slot);
            __syncthreads();
            if (k >= len) {
                x = (x + 1) % kQueues;
                ++tries;
                continue;
            }
            const int g = x + kQueues * (k / chunk);
            const int pos = (g % nch) * chunk + k % chunk;
            if (pos >= per_bh)
                continue;
            bh = g / nch;
            item = order[pos];
            return true;
        }
    }
};

__device__ inline int xcd_id()
{
    return (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kQueues - 1));  // HW_REG_XCC_ID
}

// The last workgroup to leave resets every counter for the next launch.
__device__ inline void retire_group(uint32_t *queue)
{
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned done = atomicAdd(&queue[kQueues], 1u);
        if (done == gridDim.x - 1) {
            for (int i = 0; i < kQueues; ++i)
                atomicExch(&queue[i], 0u);
            atomicExch(&queue[kQueues], 0u);
        }
    }
}

// Persistent launch: as many workgroups as can be resident, capped by the
// number of work items.
template <class Kern>
hipError_t launch_persistent(Kern kern, int threads, long long items, const AttnArgs &a, hipStream_t st)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
    if (err != hipSuccess)
        return err;
    if (per_cu < 1)
        per_cu = 1;
    long long grid = (long long)cus * per_cu;
    if (grid > items)
        grid = items;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace tra

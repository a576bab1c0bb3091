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
// `order` permutes the items inside each chunk.  A workgroup whose queue
// runs dry reads all counters at once to find the queues that still hold
// slots, so the end of a launch costs two round trips per workgroup, not
// one atomic per queue.
//
// With `tail` set, the last chunk of every queue is handed out in halves:
// its slots come twice, as (item, half 0) and (item, half 1), each half
// taking one half of the item's key blocks.  A launch with few items per
// workgroup otherwise ends with a round of whole items on some compute
// units while the others idle; halves shorten that round.  The split
// index of such a slot (queue * chunk + position in the chunk, below
// kQueues * chunk) names where the two halves meet (see the forward).
struct WorkQueue {
    uint32_t *ctr;
    const __attribute__((address_space(4))) int32_t *order;
    int per_bh, chunk, nch, total_chunks;
    bool tail;

    __device__ WorkQueue(uint32_t *queue, const int32_t *order_, int per_bh_, int chunk_, int bh_count,
                         bool tail_ = false)
        : ctr(queue), order((const __attribute__((address_space(4))) int32_t *)order_), per_bh(per_bh_),
          chunk(chunk_), nch((per_bh_ + chunk_ - 1) / chunk_), total_chunks(bh_count * nch), tail(tail_)
    {
    }

    __device__ int queue_chunks(int q) const
    {
        return total_chunks > q ? (total_chunks - q + kQueues - 1) / kQueues : 0;
    }

    // Slots of queue q (its last chunk twice over in tail mode).
    __device__ long long queue_len(int q) const
    {
        const int chunks_q = queue_chunks(q);
        return (long long)(chunks_q + (tail && chunks_q > 0 ? 1 : 0)) * chunk;
    }

    // Next item of the workgroup (wave-uniform results); false when every
    // queue is drained.  `x` is the queue being drained (start: this XCD),
    // `tries` how many queues have been found drained.  `half` is -1 for a
    // whole item, else 0 or 1 with `split` the item's split index.
    __device__ bool next(int &x, int &tries, int *slot, int &bh, int &item, int &half, int &split)
    {
        for (;;) {
            if (tries >= kQueues)
                return false;
            const long long len = queue_len(x);
            if (threadIdx.x == 0)
                *slot = (int)atomicAdd(&ctr[x], 1u);
            __syncthreads();
            const int k = __builtin_amdgcn_readfirstlane(*slot);
            __syncthreads();
            if (k >= len) {
                // Queue x is drained.  Read every queue's counter at once
                // (coherent loads, one round trip) and move to the next
                // queue after x that still has slots, instead of trying the
                // others one atomic at a time; none left ends the walk.  A
                // counter only grows, so a queue seen drained stays drained,
                // and one seen with slots is checked again by its atomic.
                ++tries;
                if (threadIdx.x < 64) {
                    const int q = threadIdx.x;
                    bool has = false;
                    if (q < kQueues)
                        has = (long long)__hip_atomic_load(&ctr[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                              queue_len(q);
                    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
                    if (threadIdx.x == 0)
                        *slot = (int)m;
                }
                __syncthreads();
                const int m = __builtin_amdgcn_readfirstlane(*slot);
                __syncthreads();
                if (m == 0)
                    return false;
                int y = x;
                for (int i = 1; i < kQueues; ++i) {
                    const int c = (x + i) % kQueues;
                    if ((m >> c) & 1) {
                        y = c;
                        break;
                    }
                }
                x = y;
                continue;
            }
            int g = x + kQueues * (k / chunk), j = k % chunk;
            half = -1;
            if (tail) {
                const int last = queue_chunks(x) - 1;
                if (k >= last * chunk) {
                    j = (k - last * chunk) >> 1;
                    half = (k - last * chunk) & 1;
                    g = x + kQueues * last;
                    split = x * chunk + j;
                }
            }
            const int pos = (g % nch) * chunk + j;
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

// Persistent launch: as many workgroups as can be resident (cached per device
// and kernel, see resident_workgroups), capped by the number of work items.
template <class Kern, class Args>
hipError_t launch_persistent(Kern kern, int threads, long long items, const Args &a, hipStream_t st)
{
    long long grid = 0;
    const hipError_t err = resident_workgroups((const void *)kern, threads, &grid);
    if (err != hipSuccess)
        return err;
    if (grid > items)
        grid = items;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace tra

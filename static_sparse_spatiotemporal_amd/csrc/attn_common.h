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

// Pop the next work item for the whole workgroup (one atomic per item).
__device__ inline int pop_item(uint32_t *queue, int *slot)
{
    if (threadIdx.x == 0)
        *slot = (int)atomicAdd(queue, 1u);
    __syncthreads();
    const int item = *slot;
    __syncthreads();
    return item;
}

// The last workgroup to leave resets the queue for the next launch.
__device__ inline void retire_group(uint32_t *queue)
{
    if (threadIdx.x == 0) {
        __threadfence();
        const unsigned done = atomicAdd(&queue[1], 1u);
        if (done == gridDim.x - 1) {
            atomicExch(&queue[0], 0u);
            atomicExch(&queue[1], 0u);
        }
    }
}

// Persistent launch: as many workgroups as can be resident, capped by the
// number of work items.
template <class Kern>
hipError_t launch_persistent(Kern kern, int threads, const AttnArgs &a, hipStream_t st)
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
    const long long items = (long long)a.B * a.H * a.mask.nqb;
    long long grid = (long long)cus * per_cu;
    if (grid > items)
        grid = items;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace tra

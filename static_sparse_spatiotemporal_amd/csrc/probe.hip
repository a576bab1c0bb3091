// Measured MFMA peak: every SIMD runs two waves of back-to-back
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic
// inside the loop, at whatever clock the chip holds under that load.  The
// benchmark reports the attention kernels against this figure beside the
// data-sheet peak.
#include "attn_common.h"
#include "probe.h"

namespace tra {
namespace {

constexpr int kProbeThreads = 512;  // 8 waves: two per SIMD
constexpr int kProbeChains = 4;     // independent accumulators per wave

__global__ __launch_bounds__(kProbeThreads) void k_mfma_loop(int64_t iters, float *out)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (lane + j));
        b[j] = (__bf16)(0.002f * (lane - j));
    }
    f32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
        acc[c] = f32x16{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sum += acc[c][i];
    // one value per workgroup keeps the loop live
    if (threadIdx.x == 0)
        out[blockIdx.x] = sum;
}

}  // namespace

int64_t mfma_loop_flops(int64_t iters, int blocks)
{
    return (int64_t)blocks * (kProbeThreads / 64) * kProbeChains * iters * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_loop(int64_t iters, int blocks, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st, iters, out);
    return hipGetLastError();
}

}  // namespace tra

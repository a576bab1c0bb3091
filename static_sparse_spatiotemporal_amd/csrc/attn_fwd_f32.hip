// fp32 attention forward (Radial Attention section 2, eq. 2) for inputs that
// must not be rounded below fp32: one thread per query row of a 128-query
// block, 16-key sub-tiles of K and V staged in LDS (every thread reads the
// same key row, an LDS broadcast), fp32 FMA dot products and an fp32
// streaming softmax in base 2.  Same mask walk and work queue as the bf16
// kernel.
#include "attn_common.h"

namespace tra {
namespace {

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_f32(AttnArgs a)
{
    constexpr int KT = 16;
    __shared__ float sK[KT][D];
    __shared__ float sV[KT][D];
    __shared__ int sItem;
    const int tid = threadIdx.x;
    const int N = a.N;
    const float c2 = a.scale_log2;

    WorkQueue wq(a.mask.queue, a.mask.order, a.mask.nqb, kChunk, a.B * a.H);
    int wx = xcd_id(), wtries = 0, bh = 0, row = 0;
    while (wq.next(wx, wtries, &sItem, bh, row)) {
        const int b = bh / a.H, h = bh - b * a.H;
        const float *Qp = (const float *)a.q + b * a.sq[0] + h * a.sq[1];
        const float *Kp = (const float *)a.k + b * a.sk[0] + h * a.sk[1];
        const float *Vp = (const float *)a.v + b * a.sv[0] + h * a.sv[1];
        float *Op = (float *)a.o + b * a.so[0] + h * a.so[1];
        const int q = row * kBlock + tid;

        float qv[D], o[D];
#pragma unroll
        for (int x = 0; x < D; ++x) {
            qv[x] = q < N ? Qp[(int64_t)q * a.sq[2] + x] : 0.f;
            o[x] = 0.f;
        }
        float m = kNegInf, l = 0.f;
        const int e0 = a.mask.row_ptr[row], e1 = a.mask.row_ptr[row + 1];
        for (int e = e0; e < e1; ++e) {
            const int kb = a.mask.col_idx[e];
            const int em = a.mask.emask_idx[e];
            uint4 mw = make_uint4(~0u, ~0u, ~0u, ~0u);
            if (em >= 0)
                mw = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + tid];
            for (int sub = 0; sub < kBlock / KT; ++sub) {
                const int key0 = kb * kBlock + sub * KT;
                __syncthreads();
                for (int u = tid; u < KT * D / 4; u += 128) {
                    const int r = u / (D / 4), c = u % (D / 4);
                    const int key = key0 + r;
                    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
                    if (key < N) {
                        kv = *(const float4 *)(Kp + (int64_t)key * a.sk[2] + 4 * c);
                        vv = *(const float4 *)(Vp + (int64_t)key * a.sv[2] + 4 * c);
                    }
                    *(float4 *)&sK[r][4 * c] = kv;
                    *(float4 *)&sV[r][4 * c] = vv;
                }
                __syncthreads();
                // bits of keys sub * KT .. sub * KT + KT - 1 of the block
                const int wsel = (sub * KT) >> 5;
                const uint32_t word = (wsel == 0 ? mw.x : wsel == 1 ? mw.y : wsel == 2 ? mw.z : mw.w)
                                      >> ((sub * KT) & 31);
                float sc[KT];
                float mx = kNegInf;
#pragma unroll 4
                for (int j = 0; j < KT; ++j) {
                    float acc = 0.f;
#pragma unroll
                    for (int x = 0; x < D; ++x)
                        acc = fmaf(qv[x], sK[j][x], acc);
                    sc[j] = ((word >> j) & 1u) ? acc * c2 : kNegInf;
                    mx = fmaxf(mx, sc[j]);
                }
                const float mnew = fmaxf(m, mx);
                const float muse = (mnew == kNegInf) ? 0.f : mnew;
                const float alpha = exp2f(m - muse);
                m = mnew;
                l *= alpha;
#pragma unroll
                for (int x = 0; x < D; ++x)
                    o[x] *= alpha;
#pragma unroll 4
                for (int j = 0; j < KT; ++j) {
                    const float p = exp2f(sc[j] - muse);
                    l += p;
#pragma unroll
                    for (int x = 0; x < D; ++x)
                        o[x] = fmaf(p, sV[j][x], o[x]);
                }
            }
        }
        if (q < N) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int x = 0; x < D; ++x)
                Op[(int64_t)q * a.so[2] + x] = o[x] * inv;
            if (a.lse)
                a.lse[(int64_t)bh * N + q] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
        }
    }

    retire_group(a.mask.queue);
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st)
{
    const long long items = (long long)a.B * a.H * a.mask.nqb;
    return a.D == 128 ? launch_persistent(attn_fwd_f32<128>, 128, items, a, st)
                      : launch_persistent(attn_fwd_f32<64>, 128, items, a, st);
}

}  // namespace tra

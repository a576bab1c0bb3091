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

// D = 64 variant with the keys of a row split over 16 lanes: a workgroup of
// 256 threads takes 16 rows of a query block; lane x of a row handles keys
// x, x + 16, .. of every kept block (K and V blocks staged in LDS with a
// one-float pad per row), keeping its own running maximum, denominator and
// output; the 16 partial softmax states of a row are merged at the end
// (max, rescale, add) with lane shuffles.
constexpr int kSplitLanes = 16;
constexpr int kSplitRows = 256 / kSplitLanes;

__global__ __launch_bounds__(256) void attn_fwd_f32_split64(AttnArgs a)
{
    constexpr int D = 64, DP = D + 1;
    __shared__ float sK[kBlock * DP];
    __shared__ float sV[kBlock * DP];
    const int tid = threadIdx.x;
    const int x = tid & (kSplitLanes - 1), rr = tid / kSplitLanes;
    const int per_bh = a.mask.nqb * (kBlock / kSplitRows);
    const int bh = blockIdx.x / per_bh, rest = blockIdx.x - bh * per_bh;
    const int qb = rest / (kBlock / kSplitRows), slice = rest - qb * (kBlock / kSplitRows);
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N;
    const float c2 = a.scale_log2;
    const float *Qp = (const float *)a.q + b * a.sq[0] + h * a.sq[1];
    const float *Kp = (const float *)a.k + b * a.sk[0] + h * a.sk[1];
    const float *Vp = (const float *)a.v + b * a.sv[0] + h * a.sv[1];
    const int r = slice * kSplitRows + rr;  // row within the query block
    const int q = qb * kBlock + r;
    float qv[D], o[D];
    const int qr = q < N ? q : N - 1;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
        const float4 v4 = *(const float4 *)(Qp + (int64_t)qr * a.sq[2] + d);
        qv[d] = v4.x * c2;
        qv[d + 1] = v4.y * c2;
        qv[d + 2] = v4.z * c2;
        qv[d + 3] = v4.w * c2;
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        o[d] = 0.f;
    float m = kNegInf, l = 0.f;
    const int e0 = a.mask.row_ptr[qb], e1 = a.mask.row_ptr[qb + 1];
    for (int e = e0; e < e1; ++e) {
        const int kb = a.mask.col_idx[e];
        const int em = a.mask.emask_idx[e];
        __syncthreads();
        for (int c = tid; c < kBlock * D / 4; c += 256) {
            const int row = c / (D / 4), col = 4 * (c % (D / 4));
            const int key = kb * kBlock + row;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (key < N) {
                kv = *(const float4 *)(Kp + (int64_t)key * a.sk[2] + col);
                vv = *(const float4 *)(Vp + (int64_t)key * a.sv[2] + col);
            }
            float *dk = sK + row * DP + col, *dv = sV + row * DP + col;
            dk[0] = kv.x; dk[1] = kv.y; dk[2] = kv.z; dk[3] = kv.w;
            dv[0] = vv.x; dv[1] = vv.y; dv[2] = vv.z; dv[3] = vv.w;
        }
        __syncthreads();
        uint4 mw = make_uint4(~0u, ~0u, ~0u, ~0u);
        if (em >= 0)
            mw = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + r];
        const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll 2
        for (int j = x; j < kBlock; j += kSplitLanes) {
            if (!((words[j >> 5] >> (j & 31)) & 1u))
                continue;
            const float *kr = sK + j * DP;
            float sc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d)
                sc = fmaf(qv[d], kr[d], sc);
            if (sc > m) {
                const float alpha = __builtin_amdgcn_exp2f(m - sc);  // m = -inf gives 0
                l *= alpha;
#pragma unroll
                for (int d = 0; d < D; ++d)
                    o[d] *= alpha;
                m = sc;
            }
            const float p = __builtin_amdgcn_exp2f(sc - m);
            l += p;
            const float *vr = sV + j * DP;
#pragma unroll
            for (int d = 0; d < D; ++d)
                o[d] = fmaf(p, vr[d], o[d]);
        }
    }
    // merge the 16 partial states of the row (lanes x ^ 1, 2, 4, 8)
#pragma unroll
    for (int off = 1; off < kSplitLanes; off <<= 1) {
        const float mo = __shfl_xor(m, off, kSplitLanes);
        const float lo = __shfl_xor(l, off, kSplitLanes);
        const float mn = fmaxf(m, mo);
        const float wa = mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float wb = mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const float other = __shfl_xor(o[d], off, kSplitLanes);
            o[d] = o[d] * wa + other * wb;
        }
        l = l * wa + lo * wb;
        m = mn;
    }
    if (q < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *orow = (float *)a.o + b * a.so[0] + h * a.so[1] + (int64_t)q * a.so[2];
        // lane x writes columns 4 x .. 4 x + 3
        float4 w4;
        w4.x = o[0] * inv;
        w4.y = o[1] * inv;
        w4.z = o[2] * inv;
        w4.w = o[3] * inv;
#pragma unroll
        for (int d = 0; d < D; d += 4)
            if (d == 4 * x) {
                w4.x = o[d] * inv;
                w4.y = o[d + 1] * inv;
                w4.z = o[d + 2] * inv;
                w4.w = o[d + 3] * inv;
            }
        *(float4 *)(orow + 4 * x) = w4;
        if (a.lse && x == 0)
            a.lse[(int64_t)bh * N + q] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st)
{
    if (a.D == 64) {
        const long long wgs = (long long)a.B * a.H * a.mask.nqb * (kBlock / kSplitRows);
        hipLaunchKernelGGL(attn_fwd_f32_split64, dim3((unsigned)wgs), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    const long long items = (long long)a.B * a.H * a.mask.nqb;
    return launch_persistent(attn_fwd_f32<128>, 128, items, a, st);
}

}  // namespace tra

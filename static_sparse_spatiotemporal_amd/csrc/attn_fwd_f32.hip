// fp32 attention forward (Radial Attention section 2, eq. 2) for inputs that
// must not be rounded below fp32: fp32 FMA dot products and an fp32
// streaming softmax in base 2, the keys of each query row split over 16
// lanes (see attn_fwd_f32_split).
#include "attn_common.h"

namespace tra {
namespace {

// Keys of a row split over 16 lanes: a workgroup of 256 threads takes 16
// rows of a query block; lane x of a row handles keys x, x + 16, .. of every
// kept block (K and V staged in LDS, rows padded to D + 4 floats and read
// as float4, KH keys per pass), keeping its own running maximum, denominator
// and output; the
// 16 partial softmax states of a row are merged at the end (max, rescale,
// add) with lane shuffles.  At D = 64 the scaled query row is held in
// registers and whole blocks are staged; at D = 128 the query row is read
// from LDS (the output alone takes 128 registers) and blocks are staged in
// 64-key halves (74 KB of LDS; 68 KB at D = 64).
constexpr int kSplitLanes = 16;
constexpr int kSplitRows = 256 / kSplitLanes;

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_split(AttnArgs a)
{
    // Rows padded to D + 4 floats: 16-byte aligned for float4 reads, and the
    // 16 lanes of a row, reading 16 consecutive keys at one column, hit 16
    // distinct 4-bank groups.
    constexpr int DP = D + 4;
    constexpr int KH = D == 64 ? kBlock : 64;  // keys staged per pass
    constexpr bool QLDS = D > 64;
    __shared__ __attribute__((aligned(16))) float sK[KH * DP];
    __shared__ __attribute__((aligned(16))) float sV[KH * DP];
    __shared__ __attribute__((aligned(16))) float sQ[QLDS ? kSplitRows * DP : 4];
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
    const int qr = q < N ? q : N - 1;
    float qv[QLDS ? 1 : D], o[D];
    if constexpr (QLDS) {
        // the 16 lanes of a row store its scaled query, D / 16 values each
        // (read after the first staging barrier)
#pragma unroll
        for (int d = 4 * x; d < D; d += 4 * kSplitLanes) {
            const float4 v4 = *(const float4 *)(Qp + (int64_t)qr * a.sq[2] + d);
            float *dq = sQ + rr * DP + d;
            dq[0] = v4.x * c2;
            dq[1] = v4.y * c2;
            dq[2] = v4.z * c2;
            dq[3] = v4.w * c2;
        }
    } else {
#pragma unroll
        for (int d = 0; d < D; d += 4) {
            const float4 v4 = *(const float4 *)(Qp + (int64_t)qr * a.sq[2] + d);
            qv[d] = v4.x * c2;
            qv[d + 1] = v4.y * c2;
            qv[d + 2] = v4.z * c2;
            qv[d + 3] = v4.w * c2;
        }
    }
    const float *qrow = sQ + rr * DP;
#pragma unroll
    for (int d = 0; d < D; ++d)
        o[d] = 0.f;
    float m = kNegInf, l = 0.f;
    const int e0 = a.mask.row_ptr[qb], e1 = a.mask.row_ptr[qb + 1];
    for (int e = e0; e < e1; ++e) {
        const int kb = a.mask.col_idx[e];
        const int em = a.mask.emask_idx[e];
        uint4 mw = make_uint4(~0u, ~0u, ~0u, ~0u);
        if (em >= 0)
            mw = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + r];
        const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
        for (int h0 = 0; h0 < kBlock; h0 += KH) {
            __syncthreads();
            for (int c = tid; c < KH * D / 4; c += 256) {
                const int row = c / (D / 4), col = 4 * (c % (D / 4));
                const int key = kb * kBlock + h0 + row;
                float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
                if (key < N) {
                    kv = *(const float4 *)(Kp + (int64_t)key * a.sk[2] + col);
                    vv = *(const float4 *)(Vp + (int64_t)key * a.sv[2] + col);
                }
                *(float4 *)(sK + row * DP + col) = kv;
                *(float4 *)(sV + row * DP + col) = vv;
            }
            __syncthreads();
#pragma unroll 2
            for (int j = x; j < KH; j += kSplitLanes) {
                const int jb = h0 + j;  // key within the block
                if (!((words[jb >> 5] >> (jb & 31)) & 1u))
                    continue;
                const float4 *kr = (const float4 *)(sK + j * DP);
                float s4[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums
#pragma unroll
                for (int d4 = 0; d4 < D / 4; ++d4) {
                    const float4 kk = kr[d4];
                    const int d = 4 * d4;
                    s4[0] = fmaf(QLDS ? qrow[d] : qv[d], kk.x, s4[0]);
                    s4[1] = fmaf(QLDS ? qrow[d + 1] : qv[d + 1], kk.y, s4[1]);
                    s4[2] = fmaf(QLDS ? qrow[d + 2] : qv[d + 2], kk.z, s4[2]);
                    s4[3] = fmaf(QLDS ? qrow[d + 3] : qv[d + 3], kk.w, s4[3]);
                }
                const float sc = (s4[0] + s4[1]) + (s4[2] + s4[3]);
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
                const float4 *vr = (const float4 *)(sV + j * DP);
#pragma unroll
                for (int d4 = 0; d4 < D / 4; ++d4) {
                    const float4 vv = vr[d4];
                    o[4 * d4] = fmaf(p, vv.x, o[4 * d4]);
                    o[4 * d4 + 1] = fmaf(p, vv.y, o[4 * d4 + 1]);
                    o[4 * d4 + 2] = fmaf(p, vv.z, o[4 * d4 + 2]);
                    o[4 * d4 + 3] = fmaf(p, vv.w, o[4 * d4 + 3]);
                }
            }
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
        // lane x writes columns 4 x .. 4 x + 3 of every 64-column group
#pragma unroll
        for (int c0 = 0; c0 < D; c0 += 4 * kSplitLanes) {
            float4 w4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int d = c0; d < c0 + 4 * kSplitLanes; d += 4)
                if (d == c0 + 4 * x) {
                    w4.x = o[d] * inv;
                    w4.y = o[d + 1] * inv;
                    w4.z = o[d + 2] * inv;
                    w4.w = o[d + 3] * inv;
                }
            *(float4 *)(orow + c0 + 4 * x) = w4;
        }
        if (a.lse && x == 0)
            a.lse[(int64_t)bh * N + q] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t st)
{
    const long long wgs = (long long)a.B * a.H * a.mask.nqb * (kBlock / kSplitRows);
    if (a.D == 64)
        hipLaunchKernelGGL(attn_fwd_f32_split<64>, dim3((unsigned)wgs), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(attn_fwd_f32_split<128>, dim3((unsigned)wgs), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace tra

// fp32 attention backward: the gradients of eq. 2 (Radial Attention section
// 2) for fp32 inputs, with fp32 arithmetic throughout.  With P the forward's
// probabilities (recomputed from Q, K and the saved LSE), dO the gradient of
// O and delta = rowsum(dO o O):
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),
//   dK = scale dS^T Q,   dQ = scale dS K.
// The fp32 workloads are small, so these kernels aim at plain, exact fp32
// work rather than matrix cores: a row is split over 16 lanes (one DPP row
// of the wave), each lane holding D / 16 of its columns; dot products are
// finished with DPP row rotations.  Three kernels, no atomics
// (deterministic):
//   k_bwd_f32_prep  per row: delta and -LSE log2(e);
//   k_bwd_f32_dq    per 16 query rows of a query block: every kept key of
//                   the block's CSR row, K and V staged in LDS 128 keys (D =
//                   64) or 64 keys (D = 128) at a time, the row's element
//                   mask read once per block;
//   k_bwd_f32_dkdv  per 16 key rows of a key block: every query block that
//                   keeps the key block (the mask's schedule over key
//                   blocks), Q, dO, -LSE log2(e), delta and the element-mask
//                   word of each query staged 128 or 64 queries at a time.
#include "attn_common.h"

namespace tra {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLanes = 16;               // lanes per row
constexpr int kRows = 256 / kLanes;      // rows per workgroup
// staged rows per step: 64 KB of LDS for the two staged operands
template <int D>
constexpr int kSubOf() { return D == 64 ? 128 : 64; }

// Sum over the 16 lanes of a row, which are one DPP row of the wave (lanes
// 16 k .. 16 k + 15): four additions of the value rotated within the row by
// 8, 4, 2 and 1 lanes (row_ror), each a single VALU instruction, where a
// lane shuffle would go through the LDS crossbar.  Every lane adds the same
// pairs of partial sums, in one order or the other, so all 16 get the same
// bits.
template <int R>
__device__ inline float row_ror_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + R, 0xf, 0xf, false));
}
__device__ inline float row_sum(float v)
{
    return row_ror_add<1>(row_ror_add<2>(row_ror_add<4>(row_ror_add<8>(v))));
}

template <int D>
__global__ __launch_bounds__(256) void k_bwd_f32_prep(BwdArgs a)
{
    constexpr int PER = D / kLanes;
    const int64_t rows = (int64_t)a.f.B * a.f.H * a.f.N;
    const int64_t r = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes;
    const int x = threadIdx.x % kLanes;
    float acc = 0.f;
    if (r < rows) {
        const int64_t bh = r / a.f.N, q = r - bh * a.f.N;
        const int64_t b = bh / a.f.H, h = bh - b * a.f.H;
        const float *o = (const float *)a.o + b * a.s_o[0] + h * a.s_o[1] + q * a.s_o[2] + x * PER;
        const float *g = (const float *)a.dout + b * a.s_do[0] + h * a.s_do[1] + q * a.s_do[2] + x * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc = fmaf(o[e], g[e], acc);
    }
    acc = row_sum(acc);
    if (r < rows && x == 0) {
        a.delta[r] = acc;
        const float l = a.lse[r];
        a.nlse[r] = l == kNegInf ? kNegInf : -l * kLog2e;
    }
}

// grid: (B * H * nqb * 128 / kRows); 16 query rows x 16 lanes.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_f32_dq(BwdArgs a)
{
    constexpr int PER = D / kLanes;
    constexpr int kSub = kSubOf<D>();
    __shared__ float sK[kSub][D];
    __shared__ float sV[kSub][D];
    const AttnArgs &f = a.f;
    const int tid = threadIdx.x, x = tid % kLanes, rr = tid / kLanes;
    const int slices = kBlock / kRows;
    const int per_bh = f.mask.nqb * slices;
    const int bh = blockIdx.x / per_bh, rest = blockIdx.x - bh * per_bh;
    const int qb = rest / slices, slice = rest - qb * slices;
    const int b = bh / f.H, h = bh - b * f.H;
    const int N = f.N;
    const float c2 = f.scale_log2, scale = c2 / kLog2e;
    const int r = slice * kRows + rr, q = qb * kBlock + r;
    const bool live = q < N;
    const int qr = live ? q : N - 1;
    const float *Qp = (const float *)f.q + b * f.sq[0] + h * f.sq[1];
    const float *Kp = (const float *)f.k + b * f.sk[0] + h * f.sk[1];
    const float *Vp = (const float *)f.v + b * f.sv[0] + h * f.sv[1];
    const float *Gp = (const float *)a.dout + b * a.s_do[0] + h * a.s_do[1];
    float qv[PER], gv[PER], dq[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        qv[e] = Qp[(int64_t)qr * f.sq[2] + x * PER + e] * c2;
        gv[e] = Gp[(int64_t)qr * a.s_do[2] + x * PER + e];
        dq[e] = 0.f;
    }
    const float nl = a.nlse[(int64_t)bh * N + qr];
    const float dl = a.delta[(int64_t)bh * N + qr];
    const int e0 = f.mask.row_ptr[qb], e1 = f.mask.row_ptr[qb + 1];
    for (int e = e0; e < e1; ++e) {
        const int kb = f.mask.col_idx[e];
        const int em = f.mask.emask_idx[e];
        // this row's element mask over the block's 128 keys, read once
        uint4 mw = make_uint4(~0u, ~0u, ~0u, ~0u);
        if (em >= 0)
            mw = ((const uint4 *)f.mask.emask)[(size_t)em * kBlock + r];
        const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
        for (int s0 = 0; s0 < kBlock; s0 += kSub) {
            const int key0 = kb * kBlock + s0;
            __syncthreads();
            for (int c = tid; c < kSub * D / 4; c += 256) {
                const int kr = c / (D / 4), col = 4 * (c - kr * (D / 4));
                const int key = key0 + kr < N ? key0 + kr : N - 1;
                *(float4 *)&sK[kr][col] = *(const float4 *)(Kp + (int64_t)key * f.sk[2] + col);
                *(float4 *)&sV[kr][col] = *(const float4 *)(Vp + (int64_t)key * f.sv[2] + col);
            }
            __syncthreads();
#pragma unroll 2
            for (int j = 0; j < kSub; ++j) {
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int e2 = 0; e2 < PER; ++e2) {
                    s = fmaf(qv[e2], sK[j][x * PER + e2], s);
                    dp = fmaf(gv[e2], sV[j][x * PER + e2], dp);
                }
                s = row_sum(s);
                dp = row_sum(dp);
                const int jb = s0 + j;
                const bool keep = live && key0 + j < N && ((words[jb >> 5] >> (jb & 31)) & 1u);
                const float p = keep ? exp2f(s + nl) : 0.f;
                const float ds = p * (dp - dl);
#pragma unroll
                for (int e2 = 0; e2 < PER; ++e2)
                    dq[e2] = fmaf(ds, sK[j][x * PER + e2], dq[e2]);
            }
        }
    }
    if (live) {
        float *dQp = (float *)a.dq + b * a.s_dq[0] + h * a.s_dq[1] + (int64_t)q * a.s_dq[2] + x * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            dQp[e] = dq[e] * scale;
    }
}

// grid: (B * H * t_npairs * 2 members * 128 / kRows); 16 key rows x 16 lanes.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_f32_dkdv(BwdArgs a)
{
    constexpr int PER = D / kLanes;
    constexpr int kSub = kSubOf<D>();
    __shared__ float sQ[kSub][D];
    __shared__ float sG[kSub][D];
    __shared__ float sL[kSub], sD[kSub];
    __shared__ uint32_t sM[kSub];  // mask word of each staged query over this workgroup's 16 keys
    const AttnArgs &f = a.f;
    const int tid = threadIdx.x, x = tid % kLanes, rr = tid / kLanes;
    const int slices = kBlock / kRows;
    const int per_bh = f.mask.t_npairs * 2 * slices;
    const int bh = blockIdx.x / per_bh, rest = blockIdx.x - bh * per_bh;
    const int pm = rest / slices, slice = rest - pm * slices;
    const int pair = pm >> 1, member = pm & 1;
    const int kb = f.mask.t_pair_cols[2 * pair + member];
    if (kb < 0)
        return;  // unpaired key block: the pair's second member is absent (whole workgroup)
    const int b = bh / f.H, h = bh - b * f.H;
    const int N = f.N;
    const float c2 = f.scale_log2, scale = c2 / kLog2e;
    const int c = slice * kRows + rr, t = kb * kBlock + c;
    const bool live = t < N;
    const int tr = live ? t : N - 1;
    const float *Qp = (const float *)f.q + b * f.sq[0] + h * f.sq[1];
    const float *Kp = (const float *)f.k + b * f.sk[0] + h * f.sk[1];
    const float *Vp = (const float *)f.v + b * f.sv[0] + h * f.sv[1];
    const float *Gp = (const float *)a.dout + b * a.s_do[0] + h * a.s_do[1];
    const float *Lp = a.nlse + (int64_t)bh * N;
    const float *Dp = a.delta + (int64_t)bh * N;
    float kv[PER], vv[PER], dk[PER], dv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        kv[e] = Kp[(int64_t)tr * f.sk[2] + x * PER + e];
        vv[e] = Vp[(int64_t)tr * f.sv[2] + x * PER + e];
        dk[e] = 0.f;
        dv[e] = 0.f;
    }
    const int u0 = f.mask.t_pair_ptr[pair], u1 = f.mask.t_pair_ptr[pair + 1];
    for (int u = u0; u < u1; ++u) {
        const int em = f.mask.t_u_em[2 * u + member];
        if (em == kAbsent)
            continue;  // uniform over the workgroup
        const int qb = f.mask.t_u_row[u];
        for (int s0 = 0; s0 < kBlock; s0 += kSub) {
            const int q0 = qb * kBlock + s0;
            __syncthreads();
            for (int i = tid; i < kSub * D / 4; i += 256) {
                const int qr = i / (D / 4), col = 4 * (i - qr * (D / 4));
                const int q = q0 + qr < N ? q0 + qr : N - 1;
                *(float4 *)&sQ[qr][col] = *(const float4 *)(Qp + (int64_t)q * f.sq[2] + col);
                *(float4 *)&sG[qr][col] = *(const float4 *)(Gp + (int64_t)q * a.s_do[2] + col);
            }
            if (tid < kSub) {
                const int q = q0 + tid < N ? q0 + tid : N - 1;
                sL[tid] = Lp[q];
                sD[tid] = Dp[q];
                // the 16 key columns of this workgroup lie in one 32-column word
                sM[tid] = em >= 0 ? f.mask.emask[((size_t)em * kBlock + s0 + tid) * 4 + ((slice * kRows) >> 5)] : ~0u;
            }
            __syncthreads();
#pragma unroll 2
            for (int i = 0; i < kSub; ++i) {
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int e2 = 0; e2 < PER; ++e2) {
                    s = fmaf(sQ[i][x * PER + e2], kv[e2], s);
                    dp = fmaf(sG[i][x * PER + e2], vv[e2], dp);
                }
                s = row_sum(s);
                dp = row_sum(dp);
                const bool keep = live && q0 + i < N && ((sM[i] >> (c & 31)) & 1u);
                const float p = keep ? exp2f(s * c2 + sL[i]) : 0.f;
                const float ds = p * (dp - sD[i]);
#pragma unroll
                for (int e2 = 0; e2 < PER; ++e2) {
                    dv[e2] = fmaf(p, sG[i][x * PER + e2], dv[e2]);
                    dk[e2] = fmaf(ds, sQ[i][x * PER + e2], dk[e2]);
                }
            }
        }
    }
    if (live) {
        float *dKp = (float *)a.dk + b * a.s_dk[0] + h * a.s_dk[1] + (int64_t)t * a.s_dk[2] + x * PER;
        float *dVp = (float *)a.dv + b * a.s_dv[0] + h * a.s_dv[1] + (int64_t)t * a.s_dv[2] + x * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            dKp[e] = dk[e] * scale;
            dVp[e] = dv[e];
        }
    }
}

template <int D>
hipError_t launch_d(const BwdArgs &a, hipStream_t st)
{
    const long long rows = (long long)a.f.B * a.f.H * a.f.N;
    hipLaunchKernelGGL(k_bwd_f32_prep<D>, dim3((unsigned)((rows + kRows - 1) / kRows)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long long bh = (long long)a.f.B * a.f.H;
    const long long dq_wgs = bh * a.f.mask.nqb * (kBlock / kRows);
    hipLaunchKernelGGL(k_bwd_f32_dq<D>, dim3((unsigned)dq_wgs), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long long kv_wgs = bh * a.f.mask.t_npairs * 2 * (kBlock / kRows);
    hipLaunchKernelGGL(k_bwd_f32_dkdv<D>, dim3((unsigned)kv_wgs), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdArgs &a, hipStream_t st)
{
    return a.f.D == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}

}  // namespace tra

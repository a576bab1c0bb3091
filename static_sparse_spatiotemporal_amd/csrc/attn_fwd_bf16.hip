// Block-sparse flash-attention forward for gfx950 (MI355X), bf16 inputs,
// fp32 accumulation.
//
// Computes O = softmax((Q K^T + M) * scale) V (Radial Attention section 2,
// eq. 2) for one 128-query block at a time over the kept 128-key blocks of
// its CSR row, with the streaming softmax: running row maximum m and
// denominator l, the accumulator rescaled by 2^(m_old - m_new) when the
// maximum grows.  Scores are multiplied by scale * log2(e) so that exp is
// v_exp_f32 (base 2).
//
// Mapping (one workgroup = 4 wave64s = one 128-query block; two workgroups
// per CU, i.e. two waves per SIMD, so one wave's softmax can run while the
// other wave's matrix products occupy the MFMA unit):
//   - wave w owns queries 32w .. 32w+31; its Q fragments stay in registers;
//   - scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane holds one query and 64 of the 128 keys
//     of the tile, so the row max is lane-local plus one permlane32 swap, and
//     the row sum stays lane-local until the epilogue;
//   - the output is accumulated transposed, O^T += V^T P^T: the probabilities
//     are already the B operand (keys permuted inside each 16-key step in
//     the same way on both operands), and V^T comes from the row-major V
//     tile through ds_read_b64_tr_b16;
//   - K and V tiles (128 x D bf16, 64 KB per workgroup at D = 128) are copied
//     HBM -> LDS by global_load_lds_dwordx4 (no register staging) with an XOR
//     swizzle of 16-byte chunks that keeps the K operand reads and the
//     transposing V reads free of bank conflicts.  The next K tile streams in
//     during softmax and P V, the next V tile during the next Q K^T;
//   - the accumulator is rescaled only when some row's maximum grows by more
//     than 2^8 (wave-uniform test); otherwise the stale maximum is kept, which
//     leaves probabilities <= 2^8 and the result exact up to rounding;
//   - partly kept tiles get their element bitmask applied to the scores;
//   - workgroups are persistent and pop (batch * head, query block) items
//     from a device counter in the mask's heaviest-first order.
#include "attn_common.h"

namespace tra {
namespace {

#define LDS_AS __attribute__((address_space(3)))

template <int D>
struct Geo {
    static constexpr int ROWB = D * 2;      // bytes per K/V row
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;    // rows per 1 KB copy instruction
    static constexpr int NCOPY = CPR / 2;   // copy instructions per thread per tile
    static constexpr int NKS = D / 16;      // k-steps of Q K^T
    static constexpr int NDB = D / 32;      // 32-row blocks of O^T
};

// Physical chunk = logical chunk XOR swizzle(row).
template <int D>
__device__ inline int k_swz(int row)
{
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ inline int v_swz(int row)
{
    return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

__device__ inline void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copy one 128-row tile of X (rows key0 ..) into LDS; rows past N repeat row
// N - 1 (their scores are masked, so only finiteness matters).
template <int D>
__device__ inline void copy_tile(const __bf16 *X, int64_t stride, int key0, int N, char LDS_AS *dst,
                                 int wave, int row0, int col)
{
    using G = Geo<D>;
    const bool whole = key0 + 128 <= N;
#pragma unroll
    for (int i = 0; i < G::NCOPY; ++i) {
        int r = key0 + row0 + 4 * G::RPI * i;
        if (!whole)
            r = r < N ? r : N - 1;
        const __bf16 *src = X + (int64_t)r * stride + col;
        __builtin_amdgcn_global_load_lds((const void *)src, (void LDS_AS *)(dst + (4 * i + wave) * 1024), 16, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(AttnArgs a)
{
    using G = Geo<D>;
    __shared__ __attribute__((aligned(1024))) char sK[kBlock * G::ROWB];
    __shared__ __attribute__((aligned(1024))) char sV[kBlock * G::ROWB];
    __shared__ int sItem;
    char LDS_AS *lK = (char LDS_AS *)sK;
    char LDS_AS *lV = (char LDS_AS *)sV;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int N = a.N, nqb = a.mask.nqb, total = a.B * a.H * nqb;
    const float c2 = a.scale_log2;
    constexpr float kTau = 8.f;

    // LDS byte offsets of this lane's operand fragments (tile-invariant).
    int koff[G::NKS];
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks)
        koff[ks] = lq * G::ROWB + (((2 * ks + hh) ^ k_swz<D>(lq)) << 4);
    int voff[G::NDB];
    {
        const int g = lane >> 4, r16 = lane & 15;
        const int keyA = 4 * hh + (r16 >> 2);
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            const int d = db * 32 + (g & 1) * 16 + 4 * (r16 & 3);
            voff[db] = keyA * G::ROWB + (((d >> 3) ^ v_swz<D>(keyA)) << 4) + ((d & 7) << 1);
        }
    }
    // Copy geometry: row of this lane in copy instruction 0, logical column.
    const int crow0 = wave * G::RPI + lane / G::CPR;
    const int cpc = lane % G::CPR;
    const int colK = (cpc ^ k_swz<D>(crow0)) * 8;
    const int colV = (cpc ^ v_swz<D>(crow0)) * 8;

    for (;;) {
        const int item = pop_item(a.mask.queue, &sItem);
        if (item >= total)
            break;
        const int bh = item / nqb;
        const int row = a.mask.order[item - bh * nqb];
        const int b = bh / a.H, h = bh - b * a.H;
        const __bf16 *Qp = (const __bf16 *)a.q + b * a.sq[0] + h * a.sq[1];
        const __bf16 *Kp = (const __bf16 *)a.k + b * a.sk[0] + h * a.sk[1];
        const __bf16 *Vp = (const __bf16 *)a.v + b * a.sv[0] + h * a.sv[1];
        __bf16 *Op = (__bf16 *)a.o + b * a.so[0] + h * a.so[1];
        const int q0 = row * kBlock + wave * 32;
        const int e0 = a.mask.row_ptr[row], e1 = a.mask.row_ptr[row + 1];

        if (e0 < e1) {
            copy_tile<D>(Kp, a.sk[2], a.mask.col_idx[e0] * kBlock, N, lK, wave, crow0, colK);
            copy_tile<D>(Vp, a.sv[2], a.mask.col_idx[e0] * kBlock, N, lV, wave, crow0, colV);
        }
        bf16x8 qf[G::NKS];
        {
            const int qr = q0 + lq < N ? q0 + lq : N - 1;
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks)
                qf[ks] = *(const bf16x8 *)(Qp + (int64_t)qr * a.sq[2] + ks * 16 + hh * 8);
        }
        f32x16 o[G::NDB];
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
            o[db] = f32x16{};
        float m = kNegInf, l = 0.f;
        wait_copies();
        __syncthreads();

        for (int e = e0; e < e1; ++e) {
            const int em = a.mask.emask_idx[e];
            // ---- S^T = K Q^T: 128 keys x 32 queries ----
            f32x16 s[4];
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
                s[kb4] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
                    const bf16x8 kf = *(const bf16x8 LDS_AS *)(lK + koff[ks] + kb4 * 32 * G::ROWB);
                    s[kb4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb4], 0, 0, 0);
                }
            // V(e) has landed and every wave is done with K(e): stream K(e+1).
            wait_copies();
            __syncthreads();
            if (e + 1 < e1)
                copy_tile<D>(Kp, a.sk[2], a.mask.col_idx[e + 1] * kBlock, N, lK, wave, crow0, colK);

            // ---- element mask of a partly kept tile ----
            if (em >= 0) {
                const uint4 mw = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + wave * 32 + lq];
                const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int bit = 8 * (i >> 2) + 4 * hh + (i & 3);
                        if (!((words[kb4] >> bit) & 1u))
                            s[kb4][i] = kNegInf;
                    }
            }
            // ---- streaming softmax (base 2) ----
            float mx = kNegInf;
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, s[kb4][i]);
            const float mt = lane_pair_max(mx) * c2;
            if (__builtin_amdgcn_ballot_w64(mt > m + kTau)) {
                const float mn = fmaxf(m, mt);
                const float alpha = __builtin_amdgcn_exp2f(m - (mn == kNegInf ? 0.f : mn));
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
                    o[db] *= alpha;
                l *= alpha;
                m = mn;
            }
            const float muse = m == kNegInf ? 0.f : m;
            // fp32 row sums (the LSE output keeps fp32 accuracy); the P V
            // product uses the probabilities rounded to bf16.
            bf16x8 pf[8];
            float ls[2] = {0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x8 pv;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    pv[x] = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][8 * (t & 1) + x], c2, -muse));
                    ls[x & 1] += pv[x];
                }
                pf[t] = __builtin_convertvector(pv, bf16x8);
            }
            l += ls[0] + ls[1];

            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int db = 0; db < G::NDB; ++db) {
                    const char LDS_AS *pa = lV + voff[db] + t * 16 * G::ROWB;
                    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)pa);
                    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(pa + 8 * G::ROWB));
                    const bf16x8 vf = __builtin_shufflevector(__builtin_bit_cast(bf16x4, va),
                                                              __builtin_bit_cast(bf16x4, vb),
                                                              0, 1, 2, 3, 4, 5, 6, 7);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], o[db], 0, 0, 0);
                }
            // K(e+1) has landed and every wave is done with V(e): stream V(e+1).
            wait_copies();
            __syncthreads();
            if (e + 1 < e1)
                copy_tile<D>(Vp, a.sv[2], a.mask.col_idx[e + 1] * kBlock, N, lV, wave, crow0, colV);
        }

        // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l) ----
        const float lt = lane_pair_sum(l);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int q = q0 + lq;
        if (q < N) {
            __bf16 *orow = Op + (int64_t)q * a.so[2];
#pragma unroll
            for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    f32x4 v;
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        v[x] = o[db][4 * i4 + x] * inv;
                    *(bf16x4 *)(orow + db * 32 + 8 * i4 + 4 * hh) = __builtin_convertvector(v, bf16x4);
                }
            if (a.lse && hh == 0)
                a.lse[(int64_t)bh * N + q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
        }
    }
    retire_group(a.mask.queue);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t st)
{
    return a.D == 128 ? launch_persistent(attn_fwd_bf16<128>, 256, a, st)
                      : launch_persistent(attn_fwd_bf16<64>, 256, a, st);
}

}  // namespace tra

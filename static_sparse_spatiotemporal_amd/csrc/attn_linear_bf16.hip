// SALAD linear branch (page "SALAD", section 2.1) for gfx950: ReLU-kernel
// linear attention over the same Q, K, V as the sparse branch,
//   O = phi(Q) (phi(K)^T V) / (phi(Q) . sum_t phi(K_t) + eps),  phi = ReLU,
// in O(N d^2) per (batch, head).  Three kernels:
//   k_lin_reduce   one workgroup per (b, h, chunk of 4096 rows): KV^T =
//                  V^T phi(K) (d x d, fp32) and z = sum_t phi(K_t) over its
//                  rows with 32x32x16 bf16 MFMAs; both operands are read
//                  transposed (ds_read_b64_tr_b16) from a four-stage LDS
//                  ring of 64-row K/V tiles (three tiles in flight);
//   k_lin_combine  sums the chunks, stores KV^T as a bf16 pair (hi + lo,
//                  about 16 significant bits) and z in fp32;
//   k_lin_apply    one workgroup per 1024 queries (four tiles of 256, the
//                  next tile's Q loaded while the current one is used):
//                  O^T = KV^T phi(Q)^T with phi(Q) as the register B operand
//                  (two MFMAs per step for hi and lo), the denominator
//                  phi(Q) . z per lane.
// The path is HBM-bound (Q, K, V read once, O written once).
#include "attn_common.h"

namespace tra {
namespace {

#define LDS_AS __attribute__((address_space(3)))

constexpr int kLinThreads = 512;  // 8 waves
constexpr int kLinChunk = 4096;   // rows per reduce workgroup
constexpr int kApplyRows = 1024;  // queries per apply workgroup (4 tiles of 256)

constexpr int kLinRows = 64;     // rows per K/V tile of the reduce kernel
constexpr int kLinStages = 4;    // tiles in the LDS ring (three in flight)

template <int D>
struct LGeo {
    static constexpr int ROWB = D * 2;
    static constexpr int TILE = kLinRows * ROWB;                 // one K or V tile
    static constexpr int CPR = D / 8;
    static constexpr int RPI = 64 / CPR;
    static constexpr int NCOPY = kLinRows * CPR / kLinThreads;   // copies per thread per tile
    static constexpr int NKS = D / 16;
    static constexpr int NDB = D / 32;
};

// Physical 16-byte chunk of logical chunk c in row `row`: c ^ lswz(row).
// The reduce kernel reads its tiles transposed (32 lanes over 4 rows 4k ..
// 4k + 3 at the 4 chunks of one aligned group), the apply kernel reads
// KV^T by rows (16 lanes over 16 rows at one chunk).  Rotating the low row
// bits keeps both free of bank conflicts (64 banks of 4 bytes): the 16 rows
// get distinct chunks and the 4 rows distinct chunk groups (at D = 64,
// where two rows share a bank line, within each row parity).
template <int D>
__device__ inline int lswz(int row)
{
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Copy a kLinRows-row tile (rows row0 .., clamped to N - 1) of X into LDS.
template <int D>
__device__ inline void lcopy_tile(const __bf16 *X, int64_t stride, int row0, int N, char LDS_AS *dst, int wave,
                                  int lane)
{
    using G = LGeo<D>;
    const int crow0 = wave * G::RPI + lane / G::CPR;
    const int col = ((lane % G::CPR) ^ lswz<D>(crow0)) * 8;
#pragma unroll
    for (int i = 0; i < G::NCOPY; ++i) {
        int r = row0 + crow0 + 8 * G::RPI * i;
        r = r < N ? r : N - 1;
        __builtin_amdgcn_global_load_lds((const void *)(X + (int64_t)r * stride + col),
                                         (void LDS_AS *)(dst + (8 * i + wave) * 1024), 16, 0, 0);
    }
}

// s_waitcnt immediate: vmcnt n (0 .. 63, split over bits 3:0 and 15:14),
// lgkmcnt 0, expcnt untouched.  The builtin form lets the compiler account
// for the wait, so it adds no drain of its own before reads of an LDS stage
// that is already complete.
constexpr int vm_lgkm_wait(int n) { return ((n >> 4) << 14) | 0x70 | (n & 15); }

// Transposed operand: 32 columns (block cb) x 16 rows 16 t + {8 (j / 4) +
// 4 (lane / 32) + j % 4}, j = 0 .. 7.
template <int D>
__device__ inline bf16x8 ltr(const char LDS_AS *tile, int lane, int t, int cb)
{
    using G = LGeo<D>;
    const int hh = lane >> 5, g = lane >> 4, r16 = lane & 15;
    const int ra = 16 * t + 4 * hh + (r16 >> 2);
    const int d = cb * 32 + (g & 1) * 16 + 4 * (r16 & 3);
    const int o0 = ra * G::ROWB + (((d >> 3) ^ lswz<D>(ra)) << 4) + ((d & 7) << 1);
    const int o1 = (ra + 8) * G::ROWB + (((d >> 3) ^ lswz<D>(ra + 8)) << 4) + ((d & 7) << 1);
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(tile + o0));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(tile + o1));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4, 5,
                                   6, 7);
}

typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));

// ReLU of 8 bf16 values (sign-magnitude: negative patterns are negative as
// int16, so an integer max with 0 clears them).
__device__ inline bf16x8 relu8(bf16x8 x)
{
    i16x8 v = __builtin_bit_cast(i16x8, x);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = v[j] > 0 ? v[j] : (short)0;
    return __builtin_bit_cast(bf16x8, v);
}

struct LinArgs {
    const void *q, *k, *v;
    void *o;
    int64_t sq[3], sk[3], sv[3], so[3];
    int32_t B, H, N, D, nchunk;
    float eps;
    float *part;      // [B * H * nchunk][D * D + D]: KV^T (dv-major) then z
    __bf16 *kv_hi;    // [B * H][D][D] KV^T
    __bf16 *kv_lo;    // [B * H][D][D] KV^T - hi
    float *z;         // [B * H][D]
};

// Wave w owns the output tiles (dv block w / 2 of D / 32, dk blocks
// NDB / 2 * (w % 2) ..) of KV^T; waves with dv block 0 also sum z.
template <int D>
__global__ __launch_bounds__(kLinThreads) void k_lin_reduce(LinArgs a)
{
    using G = LGeo<D>;
    // output tiles per wave: 2 at D = 128; 1 at D = 64 (waves 4-7 only copy)
    constexpr int NT = G::NDB * G::NDB;
    constexpr int TPW = NT >= 8 ? NT / 8 : 1;
    // ring stages (K tile, then V tile); one variable per stage so the
    // compiler tells copies into one stage from reads of another
    __shared__ __attribute__((aligned(1024))) char sT0[2 * G::TILE];
    __shared__ __attribute__((aligned(1024))) char sT1[2 * G::TILE];
    __shared__ __attribute__((aligned(1024))) char sT2[2 * G::TILE];
    __shared__ __attribute__((aligned(1024))) char sT3[2 * G::TILE];
    __shared__ __attribute__((aligned(1024))) char sT4[kLinStages > 4 ? 2 * G::TILE : 1024];
    static_assert(kLinStages == 4 || kLinStages == 5, "four or five ring stages");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hh = lane >> 5;
    const int bh = blockIdx.x / a.nchunk, chunk = blockIdx.x - bh * a.nchunk;
    const int b = bh / a.H, h = bh - b * a.H;
    const __bf16 *Kp = (const __bf16 *)a.k + b * a.sk[0] + h * a.sk[1];
    const __bf16 *Vp = (const __bf16 *)a.v + b * a.sv[0] + h * a.sv[1];
    const int N = a.N;
    const int r0 = chunk * kLinChunk;
    const int r1 = r0 + kLinChunk < N ? r0 + kLinChunk : N;
    const int ntiles = (r1 - r0 + kLinRows - 1) / kLinRows;
    // tile assignment
    const int first = wave * TPW;
    int dvb[TPW], dkb[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        dvb[x] = (first + x) / G::NDB;
        dkb[x] = (first + x) % G::NDB;
    }
    const bool owns = first < NT;               // wave-uniform
    const bool zwave = owns && (first / G::NDB) == 0;  // this wave's tiles all have dv block 0
    f32x16 acc[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x)
        acc[x] = f32x16{};
    float zs[TPW] = {};

    // stage S of the ring (S is a constant once the step loop is unrolled)
#define LIN_STAGE(S)                                                                                      \
    ((S) % kLinStages == 0   ? (char LDS_AS *)sT0                                                         \
     : (S) % kLinStages == 1 ? (char LDS_AS *)sT1                                                         \
     : (S) % kLinStages == 2 ? (char LDS_AS *)sT2                                                         \
     : (S) % kLinStages == 3 ? (char LDS_AS *)sT3                                                         \
                             : (char LDS_AS *)sT4)
    // tiles past the last one re-read the last tile (from L2) so that every
    // step issues the same copies and waits
#pragma unroll
    for (int p = 0; p < kLinStages - 1; ++p) {
        const int t = p < ntiles ? p : ntiles - 1;
        lcopy_tile<D>(Kp, a.sk[2], r0 + t * kLinRows, N, LIN_STAGE(p), wave, lane);
        lcopy_tile<D>(Vp, a.sv[2], r0 + t * kLinRows, N, LIN_STAGE(p) + G::TILE, wave, lane);
    }
    for (int u0 = 0; u0 < ntiles; u0 += kLinStages) {
        // Step u: tile u is in stage u % L, tiles u + 1 .. u + L - 2 are in
        // flight; after the barrier no wave still reads stage (u - 1) % L
        // (tile u - 1), which receives tile u + L - 1.
#pragma unroll
        for (int S = 0; S < kLinStages; ++S) {
            const int u = u0 + S;
            __builtin_amdgcn_s_waitcnt(vm_lgkm_wait((kLinStages - 2) * 2 * G::NCOPY));
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");  // no LDS access moves across the barrier
            {
                const int t = u + kLinStages - 1 < ntiles ? u + kLinStages - 1 : ntiles - 1;
                char LDS_AS *dst = LIN_STAGE(S + kLinStages - 1);
                lcopy_tile<D>(Kp, a.sk[2], r0 + t * kLinRows, N, dst, wave, lane);
                lcopy_tile<D>(Vp, a.sv[2], r0 + t * kLinRows, N, dst + G::TILE, wave, lane);
            }
            if (!owns || u >= ntiles)
                continue;
            const char LDS_AS *tK = LIN_STAGE(S);
            const char LDS_AS *tV = tK + G::TILE;
            const int rows_left = N - (r0 + u * kLinRows);  // rows past N are repeated copies
#pragma unroll
            for (int t = 0; t < kLinRows / 16; ++t) {
                bf16x8 va[TPW], kb[TPW];
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    va[x] = ltr<D>(tV, lane, t, dvb[x]);
                    kb[x] = relu8(ltr<D>(tK, lane, t, dkb[x]));
                    if (rows_left < kLinRows) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (16 * t + 8 * (j >> 2) + 4 * hh + (j & 3) >= rows_left)
                                kb[x][j] = (__bf16)0.f;
                    }
                }
#pragma unroll
                for (int x = 0; x < TPW; ++x) {
                    acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[x], kb[x], acc[x], 0, 0, 0);
                    if (zwave)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            zs[x] += (float)kb[x][j];
                }
            }
        }
    }
#undef LIN_STAGE
    __builtin_amdgcn_s_waitcnt(0);  // no copy may land after the workgroup ends
    // acc[x]: lane holds KV^T[32 dvb + 8 (i / 4) + 4 hh + i % 4][32 dkb + lane % 32]
    float *out = a.part + (int64_t)blockIdx.x * (D * D + D);
    if (!owns)
        return;
#pragma unroll
    for (int x = 0; x < TPW; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int dv = 32 * dvb[x] + 8 * (i >> 2) + 4 * hh + (i & 3);
            out[dv * D + 32 * dkb[x] + (lane & 31)] = acc[x][i];
        }
    if (zwave) {
#pragma unroll
        for (int x = 0; x < TPW; ++x) {
            const float zt = lane_pair_sum(zs[x]);
            if (hh == 0)
                out[D * D + 32 * dkb[x] + lane] = zt;
        }
    }
}

// KV^T and z of each (b, h): sum of the chunk partials.
template <int D>
__global__ __launch_bounds__(256) void k_lin_combine(LinArgs a)
{
    const int bh = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;  // element of D * D + D
    if (e >= D * D + D)
        return;
    float s = 0.f;
    for (int c = 0; c < a.nchunk; ++c)
        s += a.part[((int64_t)bh * a.nchunk + c) * (D * D + D) + e];
    if (e < D * D) {
        const __bf16 hi = (__bf16)s;
        a.kv_hi[(int64_t)bh * D * D + e] = hi;
        a.kv_lo[(int64_t)bh * D * D + e] = (__bf16)(s - (float)hi);
    } else {
        a.z[(int64_t)bh * D + (e - D * D)] = s;
    }
}

// O^T (D x 32 queries per wave) = KV^T phi(Q)^T with KV^T from LDS (row
// reads) and phi(Q) as register B operands.
template <int D>
__global__ __launch_bounds__(kLinThreads) void k_lin_apply(LinArgs a)
{
    using G = LGeo<D>;
    __shared__ __attribute__((aligned(1024))) char sHi[D * D * 2];
    __shared__ __attribute__((aligned(1024))) char sLo[D * D * 2];
    __shared__ float sZ[D];
    // per wave: its 32 x D output tile, staged for row-contiguous stores
    __shared__ __attribute__((aligned(1024))) char sO[(kLinThreads / 64) * 32 * D * 2];
    char LDS_AS *lHi = (char LDS_AS *)sHi;
    char LDS_AS *lLo = (char LDS_AS *)sLo;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    char LDS_AS *lO = (char LDS_AS *)sO + wave * 32 * G::ROWB;
    const int lq = lane & 31, hh = lane >> 5;
    const int groups = (a.N + kApplyRows - 1) / kApplyRows;
    const int bh = blockIdx.x / groups, grp = blockIdx.x - bh * groups;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N;
    // stage KV^T (hi, lo) swizzled like a D-row tile, and z
    {
        const __bf16 *hi = a.kv_hi + (int64_t)bh * D * D;
        const __bf16 *lo = a.kv_lo + (int64_t)bh * D * D;
        for (int c = threadIdx.x; c < D * G::CPR; c += kLinThreads) {
            const int row = c / G::CPR, ch = c % G::CPR;
            const int off = row * G::ROWB + ((ch ^ lswz<D>(row)) << 4);
            *(bf16x8 LDS_AS *)(lHi + off) = *(const bf16x8 *)(hi + row * D + ch * 8);
            *(bf16x8 LDS_AS *)(lLo + off) = *(const bf16x8 *)(lo + row * D + ch * 8);
        }
        if (threadIdx.x < D)
            sZ[threadIdx.x] = a.z[(int64_t)bh * D + threadIdx.x];
    }
    __syncthreads();
    const int tiles = (N + 255) / 256;
    const int tbeg = grp * (kApplyRows / 256);
    const int tend = tbeg + kApplyRows / 256 < tiles ? tbeg + kApplyRows / 256 : tiles;
    const __bf16 *Qbh = (const __bf16 *)a.q + b * a.sq[0] + h * a.sq[1];
    // raw Q of this lane's query in the current tile; the next tile's rows
    // are loaded while the current one is multiplied
    // (the tile loop is unrolled so that the loaded registers need no
    // copies between iterations)
    bf16x8 qraw[G::NKS];
    auto load_q = [&](int tile) {
        const int q = tile * 256 + wave * 32 + lq;
        const __bf16 *Qp = Qbh + (int64_t)(q < N ? q : N - 1) * a.sq[2];
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks)
            qraw[ks] = *(const bf16x8 *)(Qp + ks * 16 + hh * 8);
    };
    load_q(tbeg);
#pragma unroll
    for (int i = 0; i < kApplyRows / 256; ++i) {
        const int tile = tbeg + i;
        if (tile >= tend)
            break;
        const int q = tile * 256 + wave * 32 + lq;
        bf16x8 qf[G::NKS];
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks)
            qf[ks] = relu8(qraw[ks]);
        if (i + 1 < kApplyRows / 256 && tile + 1 < tend)
            load_q(tile + 1);
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                den = fmaf((float)qf[ks][j], sZ[ks * 16 + hh * 8 + j], den);
        den = lane_pair_sum(den);
        f32x16 o[G::NDB];
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
            o[db] = f32x16{};
        // KV^T is re-read from LDS per tile: an opaque zero keeps the reads
        // (D * D * 4 bytes per lane) from being hoisted out of the tile loop
        int rebase = 0;
        asm volatile("" : "+v"(rebase));
#pragma unroll
        for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
            for (int db = 0; db < G::NDB; ++db) {
                const int row = db * 32 + lq;
                const int off = rebase + row * G::ROWB + (((2 * ks + hh) ^ lswz<D>(row)) << 4);
                const bf16x8 ah = *(const bf16x8 LDS_AS *)(lHi + off);
                const bf16x8 al = *(const bf16x8 LDS_AS *)(lLo + off);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[ks], o[db], 0, 0, 0);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[ks], o[db], 0, 0, 0);
            }
        // O^T tile -> LDS rows (16-byte chunks XOR-swizzled by row), then
        // 16 bytes per lane, 64 / CPR rows per store.  Lanes past N computed
        // row N - 1 from the same inputs and store the same bits there; the
        // unconditional stores keep the wait for the next tile's Q at the
        // stores issued after it.
        {
            const float inv = 1.f / (den + a.eps);
#pragma unroll
            for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    f32x4 v;
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        v[x] = o[db][4 * i4 + x] * inv;
                    const int ch = (4 * db + i4) ^ (lq & (G::CPR - 1));
                    *(bf16x4 LDS_AS *)(lO + lq * G::ROWB + ch * 16 + hh * 8) = __builtin_convertvector(v, bf16x4);
                }
            const int rsub = lane / G::CPR, ch = lane % G::CPR;
#pragma unroll
            for (int i = 0; i < 32 / G::RPI; ++i) {
                const int r = i * G::RPI + rsub;
                const bf16x8 val = *(const bf16x8 LDS_AS *)(lO + r * G::ROWB + ((ch ^ (r & (G::CPR - 1))) << 4));
                const int qo = tile * 256 + wave * 32 + r;
                __bf16 *orow = (__bf16 *)a.o + b * a.so[0] + h * a.so[1] + (int64_t)(qo < N ? qo : N - 1) * a.so[2];
                *(bf16x8 *)(orow + ch * 8) = val;
            }
        }
    }
}

}  // namespace

size_t linear_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D)
{
    const int64_t nchunk = (N + kLinChunk - 1) / kLinChunk;
    const int64_t part = B * H * nchunk * (D * D + D) * 4;
    const int64_t kv = B * H * D * D * 2 * 2 + B * H * D * 4;
    return (size_t)(part + kv + 256);
}

hipError_t launch_linear_attn_bf16(const void *q, const int64_t *sq, const void *k, const int64_t *sk,
                                   const void *v, const int64_t *sv, void *o, const int64_t *so, int64_t B,
                                   int64_t H, int64_t N, int64_t D, float eps, void *ws, hipStream_t st)
{
    LinArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    for (int i = 0; i < 3; ++i) {
        a.sq[i] = sq[i];
        a.sk[i] = sk[i];
        a.sv[i] = sv[i];
        a.so[i] = so[i];
    }
    a.B = (int32_t)B;
    a.H = (int32_t)H;
    a.N = (int32_t)N;
    a.D = (int32_t)D;
    a.nchunk = (int32_t)((N + kLinChunk - 1) / kLinChunk);
    a.eps = eps;
    char *p = (char *)ws;
    a.part = (float *)p;
    p += (size_t)B * H * a.nchunk * (D * D + D) * 4;
    a.kv_hi = (__bf16 *)p;
    p += (size_t)B * H * D * D * 2;
    a.kv_lo = (__bf16 *)p;
    p += (size_t)B * H * D * D * 2;
    a.z = (float *)p;
    const unsigned red = (unsigned)(B * H * a.nchunk);
    const dim3 comb((unsigned)((D * D + D + 255) / 256), (unsigned)(B * H));
    const unsigned app = (unsigned)(B * H * ((N + kApplyRows - 1) / kApplyRows));
    if (D == 128) {
        hipLaunchKernelGGL(k_lin_reduce<128>, dim3(red), dim3(kLinThreads), 0, st, a);
        hipLaunchKernelGGL(k_lin_combine<128>, comb, dim3(256), 0, st, a);
        hipLaunchKernelGGL(k_lin_apply<128>, dim3(app), dim3(kLinThreads), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_lin_reduce<64>, dim3(red), dim3(kLinThreads), 0, st, a);
        hipLaunchKernelGGL(k_lin_combine<64>, comb, dim3(256), 0, st, a);
        hipLaunchKernelGGL(k_lin_apply<64>, dim3(app), dim3(kLinThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace tra

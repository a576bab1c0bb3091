// Block-sparse attention backward for gfx950 (MI355X), bf16 inputs, fp32
// accumulation: the gradients of eq. 2 (Radial Attention section 2) from the
// row log-sum-exp saved by the forward pass.  With P = exp(scale Q K^T + M -
// LSE) (the forward's probabilities, recomputed), dO the gradient of O and
// delta = rowsum(dO o O) = rowsum(P o dP):
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),
//   dK = scale dS^T Q,   dQ = scale dS K.
// P is recomputed from the raw dot products q.k of the bf16 inputs (fp32
// accumulation) as 2^(q.k scale log2(e) - LSE log2(e)), one fused
// multiply-add per score before v_exp_f32, so that its rows sum to 1
// against the forward's LSE.
// Three kernels, no atomics (results are deterministic):
//   k_bwd_prep   per row: delta and -LSE log2(e) (workspace);
//   k_bwd_dkdv   one workgroup per pair of key blocks (the mask's schedule
//                over key blocks), 8 waves x 32 keys; streams the Q and dO
//                tiles of every query block that keeps one of its key blocks
//                and accumulates dK and dV in registers;
//   k_bwd_dq     one workgroup per pair of query blocks (the forward's
//                schedule), 8 waves x 32 queries; streams K and V tiles and
//                accumulates dQ.
// Both main kernels recompute S and dP with v_mfma_f32_32x32x16_bf16 and
// keep the operand that stays fixed for the workgroup (K and V, or Q and dO)
// in registers; the streamed tiles are copied HBM -> LDS with
// global_load_lds_dwordx4 into double buffers (one LDS array each, named
// statically in every step), XOR-swizzled so that both the row reads
// (ds_read_b128) and the transposed reads (ds_read_b64_tr_b16) of one tile
// are free of bank conflicts (see swz).  A partly kept block's element mask
// words are loaded before the tile's wait (dQ: one 16-byte row per lane;
// dK/dV at D = 64: two words per lane, staged in the wave's own LDS words),
// never behind the next tile's copies.
#include "attn_common.h"

namespace tra {
namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
    static constexpr int ROWB = D * 2;                     // bytes per tile row
    static constexpr int TILE = kBlock * ROWB;             // bytes per 128-row tile
    static constexpr int CPR = D / 8;                      // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;                   // rows per 1 KB copy instruction
    static constexpr int NCOPY = kBlock * CPR / kThreads;  // copies per thread per tile
    static constexpr int NKS = D / 16;                     // 16-wide steps over D
    static constexpr int NDB = D / 32;                     // 32-row blocks over D
};

// Physical 16-byte chunk of logical chunk c in row `row`: c ^ swz(row).
// Every streamed tile is read both ways, so one swizzle serves both (64
// banks of 4 bytes; a row is 64 banks at D = 128, 32 at D = 64):
//   - row reads (ds_read_b128): 16 lanes read rows r .. r + 15 at one
//     logical chunk, so swz must differ over those rows (at D = 64: over
//     the rows of one parity, as two rows share a bank line);
//   - transposed reads (ds_read_b64_tr_b16): 32 lanes read 4 rows 4k ..
//     4k + 3 at the 4 chunks of one aligned group, so swz must move those
//     rows (at D = 64: the two rows of each parity) into different groups,
//     i.e. differ in bits 2-3 (bit 2).
// Both hold for the low row bits rotated: (r & 3) << 2 | (r >> 2) & 3, and
// at D = 64 ((r >> 1) & 1) << 2 | (r >> 2) & 3.  (Plain r & 15 leaves the
// 4 rows of a transposed read in one group: 4-way conflicts.)
template <int D>
__device__ inline int swz(int row)
{
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Wait for every copy into LDS.  At D = 64 with the compiler's own s_waitcnt,
// so that it knows every earlier load to have landed (the dK/dV kernel's
// mask words, loaded before the wait, are then stored to LDS without a wait
// of their own); at D = 128 in inline assembly, which the compiler does not
// see: the visible form measured 0.3-0.5% slower there.
template <int D>
__device__ inline void wait_copies()
{
    if constexpr (D == 64) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt not waited for
        asm volatile("" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

// Copy one 128-row tile (rows row0 ..) of X into LDS; rows past N repeat row
// N - 1.  Same geometry as the forward kernel's K/V copies.
template <int D>
__device__ inline void copy_tile(const __bf16 *X, int64_t stride, int row0, int N, char LDS_AS *dst, int wave,
                                 int crow0, int col, int64_t lane_off)
{
    using G = Geo<D>;
    const __bf16 *tile = X + (int64_t)row0 * stride;
    if (row0 + kBlock <= N) {
#pragma unroll
        for (int i = 0; i < G::NCOPY; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(tile + lane_off + i * (kWaves * G::RPI) * stride),
                                             (void LDS_AS *)(dst + (kWaves * i + wave) * 1024), 16, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < G::NCOPY; ++i) {
            int r = row0 + crow0 + kWaves * G::RPI * i;
            r = (r < N ? r : N - 1) - row0;
            __builtin_amdgcn_global_load_lds((const void *)(tile + (int64_t)r * stride + col),
                                             (void LDS_AS *)(dst + (kWaves * i + wave) * 1024), 16, 0, 0);
        }
    }
}

// Copy 128 floats of a per-row vector (rows row0 .., clamped to N - 1) into
// LDS; waves `w0` and `w0 + 1` each copy 64.
__device__ inline void copy_row_vec(const float *x, int row0, int N, float LDS_AS *dst, int wave, int w0, int lane)
{
    if (wave == w0 || wave == w0 + 1) {
        int r = row0 + (wave - w0) * 64 + lane;
        r = r < N ? r : N - 1;
        __builtin_amdgcn_global_load_lds((const void *)(x + r), (void LDS_AS *)(dst + (wave - w0) * 64), 4, 0, 0);
    }
}

// Byte offsets of a lane's fragments in a swizzled tile.
//   row:      A operand of 32 rows x 16 columns (rows r0 + lane % 32, columns
//             16 ks + 8 (lane / 32) ..), one ds_read_b128 per fragment;
//   tr:       A operand of 32 columns x 16 rows read transposed: rows
//             16 t + 4 (lane / 32) + (lane % 16) / 4 (+ 8 for the second
//             half), columns 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4).
template <int D>
struct TileOffsets {
    // With XOR swizzles of the low row bits, the fragment of k-step ks is
    // row0 ^ (ks << 5) and that of 32-row block db is tr0[x] ^ (db << 6)
    // (the XOR touches only bits below the row pitch), so three values per
    // lane stand for all of them.
    int row0;
    int tr0[2];
    __device__ TileOffsets(int lane)
    {
        using G = Geo<D>;
        const int lq = lane & 31, hh = lane >> 5;
        row0 = lq * G::ROWB + ((hh ^ swz<D>(lq)) << 4);
        const int g = lane >> 4, r16 = lane & 15;
        const int ra = 4 * hh + (r16 >> 2);
        const int d = (g & 1) * 16 + 4 * (r16 & 3);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int r = ra + 8 * x;
            tr0[x] = r * G::ROWB + (((d >> 3) ^ swz<D>(r)) << 4) + ((d & 7) << 1);
        }
    }
    __device__ int row(int ks) const { return row0 ^ (ks << 5); }
    __device__ int tr(int db, int x) const { return tr0[x] ^ (db << 6); }
};

// A operand (32 columns of block db x 16 rows 16 t ..) by transposed reads;
// the row order matches the probability layout of the B operands below.
template <int D>
__device__ inline bf16x8 read_tr(const char LDS_AS *tile, const TileOffsets<D> &off, int t, int db)
{
    const char LDS_AS *p = tile + t * 16 * Geo<D>::ROWB;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(p + off.tr(db, 0)));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(p + off.tr(db, 1)));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4,
                                   5, 6, 7);
}

// Store the transposed 32-row-block accumulators acc[db] (rows = D columns of
// the output, columns = the 32 rows of this wave) as row `row` of X.
template <int D>
__device__ inline void store_rows_t(__bf16 *X, int64_t stride, int row, int N, const f32x16 *acc, float mul, int hh)
{
    if (row >= N)
        return;
    __bf16 *xr = X + (int64_t)row * stride;
#pragma unroll
    for (int db = 0; db < Geo<D>::NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 v;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                v[x] = acc[db][4 * i4 + x] * mul;
            *(bf16x4 *)(xr + db * 32 + 8 * i4 + 4 * hh) = __builtin_convertvector(v, bf16x4);
        }
}

// ---------------------------------------------------------------- prep

// Per row r = (b, h, q), 8 lanes per row: delta[r] = sum_d dO[r, d] O[r, d]
// and nlse[r] = -LSE[r] log2(e) (-inf for an empty row, whose probabilities
// are then 0).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdArgs a)
{
    constexpr int PER = D / 8;  // elements per lane
    const int64_t rows = (int64_t)a.f.B * a.f.H * a.f.N;
    const int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    float acc = 0.f;
    if (r < rows) {
        const int64_t bh = r / a.f.N, q = r - bh * a.f.N;
        const int64_t b = bh / a.f.H, h = bh - b * a.f.H;
        const __bf16 *o = (const __bf16 *)a.o + b * a.s_o[0] + h * a.s_o[1] + q * a.s_o[2] + part * PER;
        const __bf16 *g = (const __bf16 *)a.dout + b * a.s_do[0] + h * a.s_do[1] + q * a.s_do[2] + part * PER;
#pragma unroll
        for (int c = 0; c < PER / 8; ++c) {
            const bf16x8 ov = *(const bf16x8 *)(o + 8 * c);
            const bf16x8 gv = *(const bf16x8 *)(g + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = fmaf((float)ov[e], (float)gv[e], acc);
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (r < rows && part == 0) {
        a.delta[r] = acc;
        const float l = a.lse[r];
        a.nlse[r] = l == kNegInf ? kNegInf : -l * kLog2e;
    }
}

// ---------------------------------------------------------------- dK, dV

// Workgroup = pair of key blocks; waves 0-3 own the first, 4-7 the second,
// 32 keys each.  Per query tile and 32-query chunk c (lane = key, 16 queries
// 32 c + 8 (i / 4) + 4 (lane / 32) + i % 4 per lane):
//   S = Q K^T and dP = dO V^T with K, V as register B operands;
//   P = 2^(S scale log2 e - LSE log2 e), dS = P (dP - delta);
//   dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read transposed
//   (dK = scale dK^T, transposed back, at the store).
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_bwd_dkdv(BwdArgs a)
{
    using G = Geo<D>;
    // double buffers, one LDS array each, named statically in every tile
    // step: the compiler then tells the copy into one buffer from the reads
    // of the other and does not wait for the next tile's copy
    __shared__ __attribute__((aligned(1024))) char sQ0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sQ1[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sO0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sO1[G::TILE];
    __shared__ __attribute__((aligned(16))) float sL0[kBlock];
    __shared__ __attribute__((aligned(16))) float sL1[kBlock];
    __shared__ __attribute__((aligned(16))) float sD0[kBlock];
    __shared__ __attribute__((aligned(16))) float sD1[kBlock];
    // D = 64: per wave, its mask word of each query row of a partly kept
    // block (D = 128 reads the words from global memory)
    constexpr bool kStageMask = D == 64;
    __shared__ __attribute__((aligned(16))) int sMw[kStageMask ? kWaves : 1][kBlock];
    __shared__ int sItem;

    const AttnArgs &f = a.f;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, w4 = wave & 3;
    const int lq = lane & 31, hh = lane >> 5;
    const int N = f.N;
    const float c2 = f.scale_log2;
    const float scale = c2 / kLog2e;

    typedef const __attribute__((address_space(4))) int32_t cint;
    cint *pair_cols = (cint *)f.mask.t_pair_cols;
    cint *pair_ptr = (cint *)f.mask.t_pair_ptr;
    cint *u_row = (cint *)f.mask.t_u_row;
    cint *u_em = (cint *)f.mask.t_u_em;

    WorkQueue wq(f.mask.queue, f.mask.t_pair_order, f.mask.t_npairs, kPairChunk, f.B * f.H);
    int wx = xcd_id(), wtries = 0, bh = 0, pair = 0;
    int whalf = -1, wsplit = 0;
    while (wq.next(wx, wtries, &sItem, bh, pair, whalf, wsplit)) {
        const int kcol = pair_cols[2 * pair + half];  // -1: this half idles
        const bool active = kcol >= 0;
        const int u0 = pair_ptr[pair], u1 = pair_ptr[pair + 1];
        const int b = bh / f.H, h = bh - b * f.H;
        const __bf16 *Qp = (const __bf16 *)f.q + b * f.sq[0] + h * f.sq[1];
        const __bf16 *Kp = (const __bf16 *)f.k + b * f.sk[0] + h * f.sk[1];
        const __bf16 *Vp = (const __bf16 *)f.v + b * f.sv[0] + h * f.sv[1];
        const __bf16 *Gp = (const __bf16 *)a.dout + b * a.s_do[0] + h * a.s_do[1];
        const float *Lp = a.nlse + (int64_t)bh * N;
        const float *Dp = a.delta + (int64_t)bh * N;
        const int key0 = kcol * kBlock + w4 * 32;

        auto copy_all = [&](int u, char LDS_AS *dQ, char LDS_AS *dO, float LDS_AS *dL, float LDS_AS *dD) {
            // copy geometry recomputed from an opaque lane (a few VALU
            // operations) rather than held in registers across the loop
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int crow0 = wave * G::RPI + ln / G::CPR;
            const int col = ((ln % G::CPR) ^ swz<D>(crow0)) * 8;
            const int r0 = u_row[u] * kBlock;
            copy_tile<D>(Qp, f.sq[2], r0, N, dQ, wave, crow0, col, crow0 * f.sq[2] + col);
            copy_tile<D>(Gp, a.s_do[2], r0, N, dO, wave, crow0, col, crow0 * a.s_do[2] + col);
            copy_row_vec(Lp, r0, N, dL, wave, 0, ln);
            copy_row_vec(Dp, r0, N, dD, wave, 2, ln);
        };
        if (u0 < u1)
            copy_all(u0, (char LDS_AS *)sQ0, (char LDS_AS *)sO0, (float LDS_AS *)sL0, (float LDS_AS *)sD0);
        // K and V rows of this lane's key as B operands (K^T, V^T fragments)
        bf16x8 kf[G::NKS], vf[G::NKS];
        if (active) {
            const int kr = key0 + lq < N ? key0 + lq : N - 1;
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks) {
                kf[ks] = *(const bf16x8 *)(Kp + (int64_t)kr * f.sk[2] + ks * 16 + hh * 8);
                vf[ks] = *(const bf16x8 *)(Vp + (int64_t)kr * f.sv[2] + ks * 16 + hh * 8);
            }
        }
        f32x16 dk[G::NDB], dv[G::NDB];
#pragma unroll
        for (int db = 0; db < G::NDB; ++db) {
            dk[db] = f32x16{};
            dv[db] = f32x16{};
        }

        // tile u is in buffer (u - u0) & 1; two tiles per trip so that each
        // step names its buffers statically
        for (int u2 = u0; u2 < u1; u2 += 2)
#pragma unroll
        for (int buf = 0; buf < 2; ++buf) {
            const int u = u2 + buf;
            if (u >= u1)
                break;
            // D = 64: a partly kept block's mask words (this wave's word of
            // query rows lane and lane + 64) are loaded under the wait for
            // tile u and stored to LDS right after it.  Read per chunk from
            // global memory instead, each word's wait also waited for the
            // next tile's copies.
            int em = kAbsent, mlo = 0, mhi = 0;
            if (kStageMask)
                em = active ? u_em[2 * u + half] : kAbsent;
            if (kStageMask && em >= 0) {
                // base taken opaque in scalar registers and the lane id
                // re-derived, so that neither is held across the loop
                typedef const __attribute__((address_space(1))) int gi32;
                gi32 *mbase = (gi32 *)f.mask.emask;
                asm volatile("" : "+s"(mbase));
                const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
                gi32 *mw = mbase + ((size_t)em * kBlock + ln) * 4 + w4;
                mlo = mw[0];
                mhi = mw[64 * 4];
            }
            wait_copies<D>();
            if (kStageMask && em >= 0) {
                // this wave's own words: no copy writes them, and its last
                // reads of them precede these stores
                sMw[wave][lane] = mlo;
                sMw[wave][64 + lane] = mhi;
            }
            __syncthreads();
            // every step issues the same copies (the item's last step
            // re-copies its tile into the free buffer), so the outstanding
            // count at each wait is the same on every path
            copy_all(u + 1 < u1 ? u + 1 : u, (char LDS_AS *)(buf == 0 ? sQ1 : sQ0),
                     (char LDS_AS *)(buf == 0 ? sO1 : sO0), (float LDS_AS *)(buf == 0 ? sL1 : sL0),
                     (float LDS_AS *)(buf == 0 ? sD1 : sD0));
            if (!kStageMask)
                em = active ? u_em[2 * u + half] : kAbsent;
            if (em == kAbsent)
                continue;
            const char LDS_AS *tQ = (const char LDS_AS *)(buf == 0 ? sQ0 : sQ1);
            const char LDS_AS *tO = (const char LDS_AS *)(buf == 0 ? sO0 : sO1);
            const float LDS_AS *tL = (const float LDS_AS *)(buf == 0 ? sL0 : sL1);
            const float LDS_AS *tD = (const float LDS_AS *)(buf == 0 ? sD0 : sD1);
            // query rows past N (repeated copies of row N - 1) must not count
            const int rows_left = N - u_row[u] * kBlock;

#pragma unroll 1
            for (int c = 0; c < 4; ++c) {
                const int cr = c * 32 * G::ROWB;
                // the fragment base offsets are recomputed per chunk (a few
                // VALU operations) instead of held in registers across the
                // loop
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const TileOffsets<D> off(ln);
                // every lane-dependent value of the chunk comes from the
                // opaque lane id too: held across the loop instead, such
                // values were spilled and reloaded after the next tile's
                // copies had been issued, and waiting for a reload then
                // waited for those copies
                const int lqc = ln & 31, hhc = ln >> 5;
                // ---- S = Q K^T, dP = dO V^T (32 queries x 32 keys) ----
                // element i of this lane is query 32 c + 8 (i / 4) + 4 hh + i % 4;
                // operand fragments are read one k-step ahead
                f32x16 s = f32x16{}, dp = f32x16{};
                bf16x8 qa[2], ga[2];
                qa[0] = *(const bf16x8 LDS_AS *)(tQ + cr + off.row(0));
                ga[0] = *(const bf16x8 LDS_AS *)(tO + cr + off.row(0));
#pragma unroll
                for (int ks = 0; ks < G::NKS; ++ks) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (ks + 1 < G::NKS) {
                        qa[(ks + 1) & 1] = *(const bf16x8 LDS_AS *)(tQ + cr + off.row(ks + 1));
                        ga[(ks + 1) & 1] = *(const bf16x8 LDS_AS *)(tO + cr + off.row(ks + 1));
                    }
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks & 1], kf[ks], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[ks & 1], vf[ks], dp, 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (kStageMask && em >= 0) {
                    // mask words of query rows 32 c + 8 g + 4 hh + j (j =
                    // 0..3), one read per g; the lane's key bit,
                    // sign-extended, selects the score or -inf
                    const int LDS_AS *mrow = (const int LDS_AS *)&sMw[wave][c * 32 + 4 * hhc];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const i32x4 words = *(const i32x4 LDS_AS *)(mrow + 8 * g);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int keep = __builtin_amdgcn_sbfe(words[j], lqc, 1);
                            s[4 * g + j] = __int_as_float((__float_as_int(s[4 * g + j]) & keep) |
                                                          (__float_as_int(kNegInf) & ~keep));
                        }
                    }
                } else if (em >= 0) {
                    // base taken opaque in scalar registers here: hoisted, it
                    // was held in (spilled) vector registers across the loop.
                    // A global (not generic) pointer: generic loads may alias
                    // LDS and were issued one at a time, each behind a wait.
                    typedef const __attribute__((address_space(1))) uint32_t gu32;
                    gu32 *mbase = (gu32 *)a.f.mask.emask;
                    asm volatile("" : "+s"(mbase));
                    gu32 *mrow = mbase + ((size_t)em * kBlock + c * 32) * 4 + w4;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int qi = 8 * (i >> 2) + 4 * hhc + (i & 3);
                        if (!((mrow[qi * 4] >> lqc) & 1u))
                            s[i] = kNegInf;
                    }
                }
                if (rows_left < kBlock) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (c * 32 + 8 * (i >> 2) + 4 * hhc + (i & 3) >= rows_left)
                            s[i] = kNegInf;
                }
                // four elements (one delta vector) at a time
                bf16x4 pq[4], sq[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 dl = *(const f32x4 LDS_AS *)(tD + c * 32 + 8 * r4 + 4 * hhc);
                    const f32x4 nl = *(const f32x4 LDS_AS *)(tL + c * 32 + 8 * r4 + 4 * hhc);
                    f32x4 pv, dsv;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int i = 4 * r4 + x;
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, nl[x]));
                        pv[x] = p;
                        dsv[x] = p * (dp[i] - dl[x]);
                    }
                    pq[r4] = __builtin_convertvector(pv, bf16x4);
                    sq[r4] = __builtin_convertvector(dsv, bf16x4);
                }
                bf16x8 pb[2], sb[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    pb[t] = __builtin_shufflevector(pq[2 * t], pq[2 * t + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                    sb[t] = __builtin_shufflevector(sq[2 * t], sq[2 * t + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                }
                // ---- dV^T += dO^T P, dK^T += Q^T dS over the 32 queries ----
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int db = 0; db < G::NDB; ++db) {
                        const bf16x8 ga = read_tr<D>(tO + cr, off, t, db);
                        const bf16x8 qa = read_tr<D>(tQ + cr, off, t, db);
                        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pb[t], dv[db], 0, 0, 0);
                        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb[t], dk[db], 0, 0, 0);
                    }
            }
        }
        if (active) {
            __bf16 *dKp = (__bf16 *)a.dk + b * a.s_dk[0] + h * a.s_dk[1];
            __bf16 *dVp = (__bf16 *)a.dv + b * a.s_dv[0] + h * a.s_dv[1];
            store_rows_t<D>(dKp, a.s_dk[2], key0 + lq, N, dk, scale, hh);
            store_rows_t<D>(dVp, a.s_dv[2], key0 + lq, N, dv, 1.f, hh);
        }
    }
    // A wave's copies land in issue order, so an item's last (repeated) copy
    // never overwrites the next item's first; only the workgroup's end waits.
    wait_copies<D>();
    retire_group(f.mask.queue);
}

// ---------------------------------------------------------------- dQ

// Workgroup = pair of query blocks (the forward's schedule); 32 queries per
// wave.  Per key tile and 64-key half (lane = query, 32 keys per lane):
//   S^T = K Q^T and dP^T = V dO^T with Q, dO as register B operands;
//   P = 2^(S scale log2 e - LSE log2 e), dS = P (dP - delta);
//   dQ^T += K^T dS^T with K^T read transposed.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_bwd_dq(BwdArgs a)
{
    using G = Geo<D>;
    // double buffers, one LDS array each (as in the dK/dV kernel)
    __shared__ __attribute__((aligned(1024))) char sK0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sK1[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sV0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sV1[G::TILE];
    __shared__ int sItem;

    const AttnArgs &f = a.f;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, w4 = wave & 3;
    const int lq = lane & 31, hh = lane >> 5;
    const int N = f.N;
    const float c2 = f.scale_log2;
    const float scale = c2 / kLog2e;
    const TileOffsets<D> off(lane);

    const int crow0 = wave * G::RPI + lane / G::CPR;
    const int cpc = lane % G::CPR;
    const int col = (cpc ^ swz<D>(crow0)) * 8;
    const int64_t offK = crow0 * f.sk[2] + col;
    const int64_t offV = crow0 * f.sv[2] + col;
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint *pair_rows = (cint *)f.mask.pair_rows;
    cint *pair_ptr = (cint *)f.mask.pair_ptr;
    cint *u_col = (cint *)f.mask.u_col;
    cint *u_em = (cint *)f.mask.u_em;

    WorkQueue wq(f.mask.queue, f.mask.pair_order, f.mask.npairs, kPairChunk, f.B * f.H);
    int wx = xcd_id(), wtries = 0, bh = 0, pair = 0;
    int whalf = -1, wsplit = 0;
    while (wq.next(wx, wtries, &sItem, bh, pair, whalf, wsplit)) {
        const int row = pair_rows[2 * pair + half];
        const bool active = row >= 0;
        const int u0 = pair_ptr[pair], u1 = pair_ptr[pair + 1];
        const int b = bh / f.H, h = bh - b * f.H;
        const __bf16 *Qp = (const __bf16 *)f.q + b * f.sq[0] + h * f.sq[1];
        const __bf16 *Kp = (const __bf16 *)f.k + b * f.sk[0] + h * f.sk[1];
        const __bf16 *Vp = (const __bf16 *)f.v + b * f.sv[0] + h * f.sv[1];
        const __bf16 *Gp = (const __bf16 *)a.dout + b * a.s_do[0] + h * a.s_do[1];
        const int q0 = row * kBlock + w4 * 32;

        if (u0 < u1) {
            copy_tile<D>(Kp, f.sk[2], u_col[u0] * kBlock, N, (char LDS_AS *)sK0, wave, crow0, col, offK);
            copy_tile<D>(Vp, f.sv[2], u_col[u0] * kBlock, N, (char LDS_AS *)sV0, wave, crow0, col, offV);
        }
        bf16x8 qf[G::NKS], gf[G::NKS];
        float nl = 0.f, dl = 0.f;
        if (active) {
            const int qr = q0 + lq < N ? q0 + lq : N - 1;
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks) {
                qf[ks] = *(const bf16x8 *)(Qp + (int64_t)qr * f.sq[2] + ks * 16 + hh * 8);
                gf[ks] = *(const bf16x8 *)(Gp + (int64_t)qr * a.s_do[2] + ks * 16 + hh * 8);
            }
            nl = a.nlse[(int64_t)bh * N + qr];
            dl = a.delta[(int64_t)bh * N + qr];
        }
        f32x16 dq[G::NDB];
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
            dq[db] = f32x16{};

        // tile u is in buffer (u - u0) & 1; two tiles per trip so that each
        // step names its buffers statically
        for (int u2 = u0; u2 < u1; u2 += 2)
#pragma unroll
        for (int buf = 0; buf < 2; ++buf) {
            const int u = u2 + buf;
            if (u >= u1)
                break;
            // the element mask word is loaded under the wait for tile u,
            // never after the next tile's copies (waiting for it there would
            // wait for them too)
            const int em = active ? u_em[2 * u + half] : kAbsent;
            uint4 mw = make_uint4(~0u, ~0u, ~0u, ~0u);
            if (em >= 0)
                mw = ((const uint4 *)f.mask.emask)[(size_t)em * kBlock + w4 * 32 + lq];
            wait_copies<D>();
            __syncthreads();
            // every step issues the same copies (the item's last step
            // re-copies its tile into the free buffer)
            {
                const int un = u + 1 < u1 ? u + 1 : u;
                copy_tile<D>(Kp, f.sk[2], u_col[un] * kBlock, N, (char LDS_AS *)(buf == 0 ? sK1 : sK0), wave,
                             crow0, col, offK);
                copy_tile<D>(Vp, f.sv[2], u_col[un] * kBlock, N, (char LDS_AS *)(buf == 0 ? sV1 : sV0), wave,
                             crow0, col, offV);
            }
            if (em == kAbsent)
                continue;
            const char LDS_AS *tK = (const char LDS_AS *)(buf == 0 ? sK0 : sK1);
            const char LDS_AS *tV = (const char LDS_AS *)(buf == 0 ? sV0 : sV1);

#pragma unroll 1
            for (int hf = 0; hf < 2; ++hf) {
                // ---- S^T = K Q^T, dP^T = V dO^T: 64 keys x 32 queries ----
                f32x16 s[2], dp[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    s[kb] = f32x16{};
                    dp[kb] = f32x16{};
                }
#pragma unroll
                for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const int ro = (2 * hf + kb) * 32 * G::ROWB + off.row(ks);
                        const bf16x8 ka = *(const bf16x8 LDS_AS *)(tK + ro);
                        const bf16x8 va = *(const bf16x8 LDS_AS *)(tV + ro);
                        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[kb], 0, 0, 0);
                        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], dp[kb], 0, 0, 0);
                    }
                // element i of s[kb] is key 32 (2 hf + kb) + 8 (i / 4) + 4 hh + i % 4
                if (em >= 0) {
                    // words selected in registers: indexed by the loop
                    // counter, a 4-word array was placed in LDS, and its
                    // store, issued after the next tile's copies, waited
                    // for them
                    const uint32_t words[2] = {hf ? mw.z : mw.x, hf ? mw.w : mw.y};
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int bit = 8 * (i >> 2) + 4 * hh + (i & 3);
                            if (!((words[kb] >> bit) & 1u))
                                s[kb][i] = kNegInf;
                        }
                }
                bf16x8 sb[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x8 dsv;
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const int i = 8 * (t & 1) + x;
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[t >> 1][i], c2, nl));
                        dsv[x] = p * (dp[t >> 1][i] - dl);
                    }
                    sb[t] = __builtin_convertvector(dsv, bf16x8);
                }
                // ---- dQ^T += K^T dS^T over the 64 keys ----
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int db = 0; db < G::NDB; ++db) {
                        const bf16x8 ka = read_tr<D>(tK, off, 4 * hf + t, db);
                        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sb[t], dq[db], 0, 0, 0);
                    }
            }
        }
        if (active) {
            __bf16 *dQp = (__bf16 *)a.dq + b * a.s_dq[0] + h * a.s_dq[1];
            store_rows_t<D>(dQp, a.s_dq[2], q0 + lq, N, dq, scale, hh);
        }
    }
    wait_copies<D>();  // the last (repeated) copy lands before the workgroup ends
    retire_group(f.mask.queue);
}

}  // namespace

BwdWorkspace bwd_workspace(int64_t B, int64_t H, int64_t N, int64_t D)
{
    const auto round = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = (size_t)(B * H * N);
    BwdWorkspace w;
    (void)D;
    w.delta = 0;
    w.nlse = round(rows * sizeof(float));
    w.bytes = w.nlse + round(rows * sizeof(float));
    return w;
}

hipError_t launch_attn_bwd_bf16(const BwdArgs &a, hipStream_t st)
{
    const long long rows = (long long)a.f.B * a.f.H * a.f.N;
    const unsigned grid = (unsigned)((rows + 31) / 32);
    if (a.f.D == 128)
        hipLaunchKernelGGL(k_bwd_prep<128>, dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_bwd_prep<64>, dim3(grid), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long long bh = (long long)a.f.B * a.f.H;
    e = a.f.D == 128 ? launch_persistent(k_bwd_dkdv<128>, kThreads, bh * a.f.mask.t_npairs, a, st)
                     : launch_persistent(k_bwd_dkdv<64>, kThreads, bh * a.f.mask.t_npairs, a, st);
    if (e != hipSuccess)
        return e;
    return a.f.D == 128 ? launch_persistent(k_bwd_dq<128>, kThreads, bh * a.f.mask.npairs, a, st)
                        : launch_persistent(k_bwd_dq<64>, kThreads, bh * a.f.mask.npairs, a, st);
}

}  // namespace tra

// Block-sparse flash-attention forward for gfx950 (MI355X), bf16 inputs,
// fp32 accumulation.
//
// Computes O = softmax((Q K^T + M) * scale) V (Radial Attention section 2,
// eq. 2) over the kept 128 x 128 blocks of the static mask, with the
// streaming softmax: running row maximum m and denominator l, the
// accumulator rescaled when the maximum grows.  The score MFMAs take the
// queries as given (exact bf16) and start from -m, the row maximum in use
// (in units of the raw dot product), instead of from 0, so that their output
// is the score relative to the maximum; one multiply by scale * log2(e) per
// score then feeds v_exp_f32 (base 2).
//
// Mapping.  One workgroup = 8 wave64s (two per SIMD) = one work item of the
// mask's pair schedule: two 128-query blocks whose kept key blocks largely
// coincide (for the radial mask: the same in-frame position in adjacent
// frames), walked over the union of their key blocks.  Waves 0-3 own the
// first query block, waves 4-7 the second; each wave owns 32 queries.  Every
// K/V tile loaded into LDS thus serves up to 256 queries.
//   - K and V tiles (128 x D bf16) are double-buffered in LDS (128 KB at
//     D = 128) and copied HBM -> LDS by global_load_lds_dwordx4 (no register
//     staging).  The copy of tile u + 1 is issued right after the single
//     barrier of tile u, so it has a whole tile of compute to land; each
//     buffer is its own LDS array, named statically in every step, so the
//     compiler does not hold the reads of tile u back until that copy has
//     landed.  An XOR swizzle of 16-byte chunks keeps the operand reads free
//     of bank conflicts;
//   - scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane holds one query and 64 of the 128 keys
//     of the tile, so the row max is lane-local plus one permlane32 swap, and
//     the row sum stays lane-local until the epilogue;
//   - the output is accumulated transposed, O^T += V^T P^T: the probabilities
//     are already the B operand (keys permuted inside each 16-key step in the
//     same way on both operands), and V^T comes from the row-major V tile
//     through ds_read_b64_tr_b16;
//   - operand fragments are read one step ahead of the MFMAs that use them;
//   - the accumulator is rescaled only when some row's maximum grows by more
//     than 2^8 (wave-uniform test); otherwise the stale maximum is kept, which
//     leaves probabilities <= 2^8 and the result exact up to rounding.  The
//     tile maximum is not even looked for once every row has one: the
//     exponentials are taken against the maximum in use and redone after a
//     rescale only when a lane's sum of them passes 2^32;
//   - partly kept tiles get their element bitmask applied to the scores; the
//     waves of a query block that does not keep a tile of the union skip it;
//   - workgroups are persistent and pop items from per-XCD queues of chunks
//     of neighbouring items (see WorkQueue), so that the workgroups sharing
//     an L2 stream largely the same K/V tiles.
#include "attn_common.h"

namespace tra {
namespace {

#define LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
// Items per resident workgroup below which the tail mode is used.
constexpr long long kTailItemsPerGroup = 16;
static_assert(kSplitLaneFloats >= 128 / 32 * 16 + 2 && kSplitRecFloats == kWaves * 64 * kSplitLaneFloats,
              "split record layout");

template <int D>
struct Geo {
    static constexpr int ROWB = D * 2;                  // bytes per K/V row
    static constexpr int TILE = kBlock * ROWB;          // bytes per K or V tile
    static constexpr int CPR = D / 8;                   // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;                // rows per 1 KB copy instruction
    static constexpr int NCOPY = kBlock * CPR / kThreads;  // copies per thread per tile
    static constexpr int NKS = D / 16;                  // k-steps of Q K^T
    static constexpr int NDB = D / 32;                  // 32-row blocks of O^T
};

// Physical chunk = logical chunk XOR swizzle(row).  K rows are read 16 at a
// time at one chunk column (S^T A operand); V rows 4 at a time, 64
// contiguous bytes each (ds_read_b64_tr_b16 for the V^T A operand).
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

// Relaxed agent-scope accesses of the split records (see the tail mode).
__device__ inline void store_agent(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float load_agent(float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Copy one 128-row tile of X (rows key0 ..) into LDS.  Copy instruction i of
// wave w fills bytes (8 i + w) KB .. of the tile: rows crow0 + 8 RPI i, where
// crow0 = w RPI + lane / CPR.  `lane_off` is this lane's element offset
// inside the tile (row crow0, swizzled column `col`).  Rows past N repeat row
// N - 1 (their scores are masked, so only finiteness matters).
template <int D>
__device__ inline void copy_tile(const __bf16 *X, int64_t stride, int key0, int N, char LDS_AS *dst,
                                 int wave, int crow0, int col, int64_t lane_off)
{
    using G = Geo<D>;
    const __bf16 *tile = X + (int64_t)key0 * stride;  // wave-uniform
    if (key0 + kBlock <= N) {
#pragma unroll
        for (int i = 0; i < G::NCOPY; ++i)
            __builtin_amdgcn_global_load_lds((const void *)(tile + lane_off + i * (8 * G::RPI) * stride),
                                             (void LDS_AS *)(dst + (8 * i + wave) * 1024), 16, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < G::NCOPY; ++i) {
            int r = key0 + crow0 + 8 * G::RPI * i;
            r = (r < N ? r : N - 1) - key0;
            __builtin_amdgcn_global_load_lds((const void *)(tile + (int64_t)r * stride + col),
                                             (void LDS_AS *)(dst + (8 * i + wave) * 1024), 16, 0, 0);
        }
    }
}

template <int D, bool STREAM, bool TAIL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(AttnArgs a)
{
    using G = Geo<D>;
    // Double buffers, one LDS array each: with the buffer named statically
    // in every tile step, the compiler can tell the copy into one buffer
    // from the operand reads of the other and does not wait for the next
    // tile's copy before reading the current one.
    __shared__ __attribute__((aligned(1024))) char sK0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sK1[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sV0[G::TILE];
    __shared__ __attribute__((aligned(1024))) char sV1[G::TILE];
    __shared__ int sItem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, w4 = wave & 3;
    const int lq = lane & 31, hh = lane >> 5;
    const int N = a.N;
    const float c2 = a.scale_log2;
    // rescale only when a row maximum grows by more than 2^8 in the
    // probabilities, i.e. by 8 / c2 in raw dot-product units
    const float tau = 8.f / c2;
    // At D = 128 the score chains' start (-muse in all 16 elements) stays in
    // registers for the whole item and is rebuilt only when muse moves, not
    // splatted every tile (-0.6% at n = 131072); at D = 64 those registers
    // hold the scores the lazy maximum keeps.
    constexpr bool kKeepSeed = D == 128;

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
    // Copy geometry (see copy_tile).
    const int crow0 = wave * G::RPI + lane / G::CPR;
    const int cpc = lane % G::CPR;
    const int colK = (cpc ^ k_swz<D>(crow0)) * 8;
    const int colV = (cpc ^ v_swz<D>(crow0)) * 8;
    const int64_t offK = crow0 * a.sk[2] + colK;
    const int64_t offV = crow0 * a.sv[2] + colV;
    // The schedule is read-only for the whole launch: read it through the
    // constant address space so that the loads are scalar.
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint *pair_rows = (cint *)a.mask.pair_rows;
    cint *pair_ptr = (cint *)a.mask.pair_ptr;
    cint *u_col = (cint *)a.mask.u_col;
    cint *u_em = (cint *)a.mask.u_em;

    // One work item: query block `row` of this half (-1: idle) over the key
    // blocks of schedule entries u0 .. u1 - 1.  tslot >= 0: half tslot & 1
    // of a split item (tail mode), merged through split record tslot >> 1.
    auto item = [&](int bh, int row, int u0, int u1, int split, int tslot) {
        const bool active = row >= 0;
        const int b = bh / a.H, h = bh - b * a.H;
        const __bf16 *Qp = (const __bf16 *)a.q + b * a.sq[0] + h * a.sq[1];
        const __bf16 *Kp = (const __bf16 *)a.k + b * a.sk[0] + h * a.sk[1];
        const __bf16 *Vp = (const __bf16 *)a.v + b * a.sv[0] + h * a.sv[1];
        __bf16 *Op = (__bf16 *)a.o + b * a.so[0] + h * a.so[1];
        const int q0 = row * kBlock + w4 * 32;

        auto kcol = [&](int u) { return STREAM ? u : u_col[u]; };
        if (u0 < u1) {
            copy_tile<D>(Kp, a.sk[2], kcol(u0) * kBlock, a.Nk, (char LDS_AS *)sK0, wave, crow0, colK, offK);
            copy_tile<D>(Vp, a.sv[2], kcol(u0) * kBlock, a.Nk, (char LDS_AS *)sV0, wave, crow0, colV, offV);
        }
        bf16x8 qf[G::NKS];
        if (active) {
            const int qr = q0 + lq < N ? q0 + lq : N - 1;
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks)
                qf[ks] = *(const bf16x8 *)(Qp + (int64_t)qr * a.sq[2] + ks * 16 + hh * 8);
        }
        f32x16 o[G::NDB];
#pragma unroll
        for (int db = 0; db < G::NDB; ++db)
            o[db] = f32x16{};
        // m: row maximum of the raw dot products q.k, l: row sum of
        // 2^((q.k - muse) c2); muse: the maximum the scores are taken
        // relative to (0 while m is -inf).
        float m = kNegInf, l = 0.f, muse = 0.f;
        f32x16 seed = f32x16{};

        // Tile u is in buffer (u - u0) & 1; the loop takes two tiles per
        // trip so that the buffer of each step is a constant.
        for (int u2 = u0; u2 < u1; u2 += 2)
#pragma unroll
        for (int buf = 0; buf < 2; ++buf) {
            const int u = u2 + buf;
            if (u >= u1)
                break;
            // The element mask word of a partly kept tile is loaded under the
            // wait for tile u, never after the next tile's copies.
            const int em = active ? (STREAM ? -1 : u_em[2 * u + half]) : kAbsent;
            uint4 mw = {0u, 0u, 0u, 0u};
            if (em >= 0)
                mw = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + w4 * 32 + lq];
            // Tile u has landed everywhere and every wave is done with tile
            // u - 1, whose buffer now receives tile u + 1.
            wait_copies();
            __syncthreads();
            // Every step issues the same copies (the last one of the item
            // re-copies tile u into the free buffer), so the outstanding
            // count at each wait is the same on every path and the
            // compiler's waits stay exact.
            {
                const int un = u + 1 < u1 ? u + 1 : u;
                char LDS_AS *nK = (char LDS_AS *)(buf == 0 ? sK1 : sK0);
                char LDS_AS *nV = (char LDS_AS *)(buf == 0 ? sV1 : sV0);
                copy_tile<D>(Kp, a.sk[2], kcol(un) * kBlock, a.Nk, nK, wave, crow0, colK, offK);
                copy_tile<D>(Vp, a.sv[2], kcol(un) * kBlock, a.Nk, nV, wave, crow0, colV, offV);
            }
            if (em == kAbsent)
                continue;
            const char LDS_AS *tK = (const char LDS_AS *)(buf == 0 ? sK0 : sK1);
            const char LDS_AS *tV = (const char LDS_AS *)(buf == 0 ? sV0 : sV1);

            // ---- S^T = K Q^T - muse: 128 keys x 32 queries (raw dot products) ----
            f32x16 s[4];
            const f32x16 s0 = kKeepSeed ? seed : f32x16{} - muse;
            bf16x8 kf[2][4];
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
                kf[0][kb4] = *(const bf16x8 LDS_AS *)(tK + koff[0] + kb4 * 32 * G::ROWB);
#pragma unroll
            for (int ks = 0; ks < G::NKS; ++ks) {
                __builtin_amdgcn_sched_barrier(0);
                if (ks + 1 < G::NKS) {
#pragma unroll
                    for (int kb4 = 0; kb4 < 4; ++kb4)
                        kf[(ks + 1) & 1][kb4] = *(const bf16x8 LDS_AS *)(tK + koff[ks + 1] + kb4 * 32 * G::ROWB);
                }
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4)
                    s[kb4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks & 1][kb4], qf[ks], ks == 0 ? s0 : s[kb4],
                                                                     0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- element mask of a partly kept tile ----
            if (em >= 0) {
                // element i of 32-key step kb4 is key 8 (i / 4) + 4 hh + i % 4:
                // its bit, sign-extended, selects the score or -inf
                const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
                    const int w = (int)(words[kb4] >> (4 * hh));
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int keep = __builtin_amdgcn_sbfe(w, 8 * (i >> 2) + (i & 3), 1);
                        s[kb4][i] = __int_as_float((__float_as_int(s[kb4][i]) & keep) |
                                                   (__float_as_int(kNegInf) & ~keep));
                    }
                }
            }
            // ---- streaming softmax (base 2) ----
            // Once every row of the wave has a finite maximum, a tile's
            // probabilities are first taken against the maximum in use
            // without looking for the tile's own maximum; only if some lane's
            // sum of them passes 2^32 (a score more than 26 above the
            // maximum, in log2 units) is the maximum taken and the tile's
            // exponentials redone.  Probabilities up to 2^32 leave bf16 and
            // the fp32 sums far from overflow, and the result is the same
            // up to rounding.  At D = 64 the scores stay in registers for the
            // redo; at D = 128 they do not fit beside the probabilities, and
            // the redo recomputes them from the tile, which is still in LDS.
            const bool lazy = !__builtin_amdgcn_ballot_w64(m == kNegInf);
            auto take_max = [&]() {
                float mx = kNegInf;
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        mx = fmaxf(mx, s[kb4][i]);
                const float mt = lane_pair_max(mx) + muse;
                if (__builtin_amdgcn_ballot_w64(mt > m + tau)) {
                    const float mn = fmaxf(m, mt);
                    const float alpha = __builtin_amdgcn_exp2f((m - (mn == kNegInf ? 0.f : mn)) * c2);
#pragma unroll
                    for (int db = 0; db < G::NDB; ++db)
                        o[db] *= alpha;
                    l *= alpha;
                    m = mn;
                    // re-base this tile's scores on the new maximum
                    const float mu = m == kNegInf ? 0.f : m;
                    const float dm = mu - muse;
                    muse = mu;
                    if (kKeepSeed)
                        seed = f32x16{} - muse;
#pragma unroll
                    for (int kb4 = 0; kb4 < 4; ++kb4)
                        s[kb4] -= dm;
                }
            };
            // fp32 row sums (the LSE output keeps fp32 accuracy); the P V
            // product uses the probabilities rounded to bf16.
            bf16x8 pf[8];
            float ls[2];
            auto exps = [&]() {
                ls[0] = ls[1] = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    f32x8 pv;
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        pv[x] = __builtin_amdgcn_exp2f(s[t >> 1][8 * (t & 1) + x] * c2);
                        ls[x & 1] += pv[x];
                    }
                    pf[t] = __builtin_convertvector(pv, bf16x8);
                }
            };
            if (!lazy)
                take_max();
            exps();
            if (lazy && __builtin_amdgcn_ballot_w64(!(ls[0] + ls[1] <= 0x1p32f))) {
                if constexpr (D == 128) {
                    // scores and element mask again, as above (this path is
                    // rare, so its operand reads are not pipelined)
#pragma unroll
                    for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
                        for (int kb4 = 0; kb4 < 4; ++kb4) {
                            const bf16x8 kk = *(const bf16x8 LDS_AS *)(tK + koff[ks] + kb4 * 32 * G::ROWB);
                            s[kb4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qf[ks], ks == 0 ? s0 : s[kb4],
                                                                             0, 0, 0);
                        }
                    if (em >= 0) {
                        const uint4 mr = ((const uint4 *)a.mask.emask)[(size_t)em * kBlock + w4 * 32 + lq];
                        const uint32_t words[4] = {mr.x, mr.y, mr.z, mr.w};
#pragma unroll
                        for (int kb4 = 0; kb4 < 4; ++kb4) {
                            const int w = (int)(words[kb4] >> (4 * hh));
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int keep = __builtin_amdgcn_sbfe(w, 8 * (i >> 2) + (i & 3), 1);
                                s[kb4][i] = __int_as_float((__float_as_int(s[kb4][i]) & keep) |
                                                           (__float_as_int(kNegInf) & ~keep));
                            }
                        }
                    }
                }
                take_max();
                exps();
            }
            l += ls[0] + ls[1];

            // ---- O^T += V^T P^T ----
            auto read_v = [&](int t, int db) {
                const char LDS_AS *pa = tV + voff[db] + t * 16 * G::ROWB;
                const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)pa);
                const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(pa + 8 * G::ROWB));
                return __builtin_shufflevector(__builtin_bit_cast(bf16x4, va), __builtin_bit_cast(bf16x4, vb),
                                               0, 1, 2, 3, 4, 5, 6, 7);
            };
            bf16x8 vf[2][G::NDB];
#pragma unroll
            for (int db = 0; db < G::NDB; ++db)
                vf[0][db] = read_v(0, db);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                __builtin_amdgcn_sched_barrier(0);
                if (t + 1 < 8) {
#pragma unroll
                    for (int db = 0; db < G::NDB; ++db)
                        vf[(t + 1) & 1][db] = read_v(t + 1, db);
                }
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t & 1][db], pf[t], o[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- tail mode: the two halves of a split item meet ----
        // Each half leaves m, its lane sums and its unnormalised O^T
        // fragments (each lane its own registers, so the other half reads
        // them back in the same order); the first to finish then leaves, and
        // the second takes the other's state in, both rescaled to the larger
        // maximum, and writes the output.  The sum is taken in half order,
        // not finishing order, so the output does not depend on which half
        // ends first.  The halves may run on different XCDs, whose L2s are
        // not coherent for ordinary accesses: the records are written and
        // read with agent-scope atomic accesses, which reach the coherence
        // point one by one.  An agent-scope fence would instead write back
        // and invalidate the whole L2, throwing away the K/V tiles the
        // XCD's other workgroups are streaming.
        if (TAIL && tslot >= 0) {
            constexpr int F = G::NDB * 16;
            const int rslot = tslot >> 1;
            const bool first_half = (tslot & 1) == 0;
            // each half leaves its state in its own record (record tslot);
            // the second reads the other's (tslot ^ 1)
            float *rec = a.mask.split_ws + (int64_t)tslot * kSplitRecFloats + (int64_t)wave * 64 * kSplitLaneFloats;
            if (active) {
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        f32x4 v;
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            v[x] = o[db][4 * i4 + x];
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            store_agent(rec + ((db * 4 + i4) * 4 + x) * 64 + lane, v[x]);
                    }
                store_agent(rec + F * 64 + lane, m);
                store_agent(rec + (F + 1) * 64 + lane, l);
            }
            // every wave's record stores (and its last tile copy) complete
            // before the counter moves
            wait_copies();
            __syncthreads();
            if (tid == 0)
                sItem = (int)__hip_atomic_fetch_add(&a.mask.split_ctr[rslot], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int other_done = __builtin_amdgcn_readfirstlane(sItem);
            __syncthreads();
            if (other_done == 0)
                return;
            if (tid == 0)
                __hip_atomic_store(&a.mask.split_ctr[rslot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            rec = a.mask.split_ws + (int64_t)(tslot ^ 1) * kSplitRecFloats + (int64_t)wave * 64 * kSplitLaneFloats;
            if (active) {
                const float mo = load_agent(rec + F * 64 + lane), lo = load_agent(rec + (F + 1) * 64 + lane);
                const float m0 = first_half ? m : mo, m1 = first_half ? mo : m;
                const float l0 = first_half ? l : lo, l1 = first_half ? lo : l;
                const float mn = fmaxf(m0, m1);
                const float mb = mn == kNegInf ? 0.f : mn;
                const float a0 = m0 == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m0 - mb) * c2);
                const float a1 = m1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f((m1 - mb) * c2);
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const float v = load_agent(rec + ((db * 4 + i4) * 4 + x) * 64 + lane);
                            const float o0 = first_half ? o[db][4 * i4 + x] : v;
                            const float o1 = first_half ? v : o[db][4 * i4 + x];
                            o[db][4 * i4 + x] = __builtin_fmaf(o1, a1, o0 * a0);
                        }
                    }
                l = __builtin_fmaf(l1, a1, l0 * a0);
                m = mn;
            }
        }

        // ---- epilogue: O = acc / l, LSE = ln 2 * (m c2 + log2 l) ----
        if (STREAM && active) {
            // normalised partial output and log2-sum-exp of this key split
            const float lt = lane_pair_sum(l);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int q = q0 + lq;
            if (q < N) {
                const int64_t r = ((int64_t)split * a.B * a.H + bh) * N + q;
                float *prow = a.part_o + r * D;
#pragma unroll
                for (int db = 0; db < G::NDB; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        f32x4 v;
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            v[x] = o[db][4 * i4 + x] * inv;
                        *(f32x4 *)(prow + db * 32 + 8 * i4 + 4 * hh) = v;
                    }
                if (hh == 0)
                    a.part_lse[r] = lt > 0.f ? m * c2 + __log2f(lt) : kNegInf;
            }
        } else if (active) {
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
                    a.lse[(int64_t)bh * N + q] = lt > 0.f ? (m * c2 + __log2f(lt)) * kLn2 : kNegInf;
            }
        }
    };

    if constexpr (STREAM) {
        const int it = blockIdx.x;
        const int split = it % a.nsplit, rest = it / a.nsplit;
        const int pair = rest % a.stream_pairs, bh = rest / a.stream_pairs;
        const int row = 2 * pair + half < a.mask.nqb ? 2 * pair + half : -1;
        const int u0 = split * a.split_tiles;
        const int u1 = u0 + a.split_tiles < a.nkv_tiles ? u0 + a.split_tiles : a.nkv_tiles;
        item(bh, row, u0, u1, split, -1);
        wait_copies();  // the last step's copy must land before the workgroup ends
    } else {
        WorkQueue wq(a.mask.queue, a.mask.pair_order, a.mask.npairs, kPairChunk, a.B * a.H, TAIL);
        int wx = xcd_id(), wtries = 0, bh = 0, pair = 0, whalf = -1, wsplit = 0;
        while (wq.next(wx, wtries, &sItem, bh, pair, whalf, wsplit)) {
            int u0 = pair_ptr[pair], u1 = pair_ptr[pair + 1], tslot = -1;
            if (TAIL && whalf >= 0) {
                // a half of the queue's last chunk: an item too short to
                // split runs whole as half 0
                if (u1 - u0 >= a.split_min) {
                    const int mid = u0 + (u1 - u0) / 2;
                    if (whalf == 0)
                        u1 = mid;
                    else
                        u0 = mid;
                    tslot = 2 * wsplit + whalf;
                } else if (whalf == 1) {
                    continue;
                }
            }
            item(bh, pair_rows[2 * pair + half], u0, u1, 0, tslot);
        }
        // The last step of an item re-copies its tile into the free buffer.
        // A wave's copies land in issue order, so the next item's first copy
        // still wins; only the workgroup's end has to wait for the last one.
        wait_copies();
        retire_group(a.mask.queue);
    }
}

// Merge of the key splits: per row, LSE2 = log2 sum_x 2^lse2_x and
// O = sum_x 2^(lse2_x - LSE2) O_x.  8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void k_merge_splits(AttnArgs a)
{
    constexpr int PER = D / 8;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    if (r >= rows)
        return;
    // both split loops are unrolled so that the loads of several splits are
    // in flight together (the merge is latency-bound)
    float mx = kNegInf;
#pragma unroll 8
    for (int x = 0; x < a.nsplit; ++x)
        mx = fmaxf(mx, a.part_lse[(int64_t)x * rows + r]);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        acc[e] = 0.f;
    float tot = 0.f;
#pragma unroll 4
    for (int x = 0; x < a.nsplit; ++x) {
        const float w = __builtin_amdgcn_exp2f(a.part_lse[(int64_t)x * rows + r] - mx);
        tot += w;
        const float *po = a.part_o + ((int64_t)x * rows + r) * D + part * PER;
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
            const f32x4 v = *(const f32x4 *)(po + e);
#pragma unroll
            for (int y = 0; y < 4; ++y)
                acc[e + y] = fmaf(w, v[y], acc[e + y]);
        }
    }
    const float inv = 1.f / tot;
    const int64_t bh = r / a.N, q = r - bh * a.N;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    __bf16 *orow = (__bf16 *)a.o + b * a.so[0] + h * a.so[1] + q * a.so[2] + part * PER;
#pragma unroll
    for (int e = 0; e < PER; e += 8) {
        f32x8 v;
#pragma unroll
        for (int y = 0; y < 8; ++y)
            v[y] = acc[e + y] * inv;
        *(bf16x8 *)(orow + e) = __builtin_convertvector(v, bf16x8);
    }
    if (a.lse && part == 0)
        a.lse[r] = (mx + __log2f(tot)) * kLn2;
}

// dst[b, h, row0 + r, :] = src[b, h, r, :]; one 16-byte chunk per thread.
struct RingCopy {
    const __bf16 *src;
    int64_t s[3];  // B, H, row strides of the source view
    __bf16 *ring;
};

// blockIdx.y = 0 copies K, 1 copies V (one launch per appended frame).
__global__ __launch_bounds__(256) void k_ring_copy(RingCopy k, RingCopy v, int64_t H, int64_t rows, int64_t D,
                                                  int64_t ring_rows, int64_t row0, int64_t total)
{
    const RingCopy &c = blockIdx.y == 0 ? k : v;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    const int64_t cpr = D / 8;
    const int64_t ch = t % cpr, rr = t / cpr;
    const int64_t r = rr % rows, bh = rr / rows;
    const int64_t b = bh / H, h = bh - b * H;
    const bf16x8 val = *(const bf16x8 *)(c.src + b * c.s[0] + h * c.s[1] + r * c.s[2] + 8 * ch);
    *(bf16x8 *)(c.ring + (bh * ring_rows + row0 + r) * D + 8 * ch) = val;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a_in, hipStream_t st)
{
    AttnArgs a = a_in;
    const long long items = (long long)a.B * a.H * a.mask.npairs;
    const void *kern =
        a.D == 128 ? (const void *)attn_fwd_bf16<128, false, false> : (const void *)attn_fwd_bf16<64, false, false>;
    long long grid = 0;
    const hipError_t e = resident_workgroups(kern, kThreads, &grid);
    if (e != hipSuccess)
        return e;
    // Few items per workgroup, some long enough to split: the launch would
    // end with a round of whole items on some compute units while the rest
    // idle, so the queues' last chunks run as halves.  With many items that
    // round is short anyway.
    a.tail_split = items < kTailItemsPerGroup * grid && a.max_pair_tiles >= a.split_min ? 1 : 0;
    if (a.tail_split)
        return a.D == 128 ? launch_persistent(attn_fwd_bf16<128, false, true>, kThreads, items, a, st)
                          : launch_persistent(attn_fwd_bf16<64, false, true>, kThreads, items, a, st);
    return a.D == 128 ? launch_persistent(attn_fwd_bf16<128, false, false>, kThreads, items, a, st)
                      : launch_persistent(attn_fwd_bf16<64, false, false>, kThreads, items, a, st);
}

hipError_t launch_attn_stream_bf16(const AttnArgs &a, hipStream_t st)
{
    const long long items = (long long)a.B * a.H * a.stream_pairs * a.nsplit;
    if (a.D == 128)
        hipLaunchKernelGGL((attn_fwd_bf16<128, true, false>), dim3((unsigned)items), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((attn_fwd_bf16<64, true, false>), dim3((unsigned)items), dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long long rows = (long long)a.B * a.H * a.N;
    const unsigned grid = (unsigned)((rows + 31) / 32);
    if (a.D == 128)
        hipLaunchKernelGGL(k_merge_splits<128>, dim3(grid), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_merge_splits<64>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_ring_copy(const void *k_src, const int64_t *s_k, void *ring_k, const void *v_src,
                            const int64_t *s_v, void *ring_v, int64_t B, int64_t H, int64_t rows, int64_t D,
                            int64_t ring_rows, int64_t row0, hipStream_t st)
{
    const int64_t total = B * H * rows * (D / 8);
    if (total == 0)
        return hipSuccess;
    RingCopy k{(const __bf16 *)k_src, {s_k[0], s_k[1], s_k[2]}, (__bf16 *)ring_k};
    RingCopy v{(const __bf16 *)v_src, {s_v[0], s_v[1], s_v[2]}, (__bf16 *)ring_v};
    hipLaunchKernelGGL(k_ring_copy, dim3((unsigned)((total + 255) / 256), 2), dim3(256), 0, st, k, v, H, rows, D,
                       ring_rows, row0, total);
    return hipGetLastError();
}

}  // namespace tra

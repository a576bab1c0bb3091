// Mask builder: compiles a static spatiotemporal mask into 128 x 128 block
// form (block classes, CSR of kept key blocks, element bitmasks of partly
// kept blocks, block bitmap).
//
// Every family keeps, for one query token and one key frame, a small number
// of contiguous key runs:
//   - Radial Attention section 3 eq. 4: between query frame i and key frame
//     j (r = floor(log2(max(|i-j|, 1)))) the kept keys of query position k
//     are the positions l with |k-l| <= floor(s / 2^r) - 1 while 2^r <= s
//     (the band of section 3.2, width floor(s / 2^r)), otherwise the single
//     position l = k when |i-j| is a multiple of ceil(2^r / s);
//   - Token Radius Attention: one run of 2 r_s + 1 columns per grid row
//     within r_s and per frame within r_t, cut at the grid edge;
//   - Vera 1.1 temporal module section 2.2: one run covering the frames
//     max(0, i - W + 1) .. i;
//   - sink frames (the "sink" of Radial Attention section 4's count): one
//     run over the first sink_frames frames, for every query and family.
// The builder counts and sets bits run by run instead of testing every
// element, so one thread handles one (query token, key block) pair.
//
// TRA_GRAN_BLOCK_EQ4 reads section 6's block sparsity the other way: the
// 128 x 128 blocks form a video of f frames with s / 128 blocks per frame and
// eq. 4 keeps or drops whole blocks; the element runs still give the
// element-predicate counts of the statistics.
#include "tra_internal.h"

namespace tra {
namespace {

__device__ inline int imin(int a, int b) { return a < b ? a : b; }
__device__ inline int imax(int a, int b) { return a > b ? a : b; }

// eq. 4 for one (query, key) index pair with s positions per frame.  Used on
// block indices; the token form is the run walk below.
__device__ inline bool radial_keep(int s, int q, int t)
{
    const int i = q / s, k = q - i * s, j = t / s, l = t - j * s;
    const int delta = i > j ? i - j : j - i;
    const int r = 31 - __clz(delta > 1 ? delta : 1);
    const long long p2 = 1ll << r;
    if (p2 <= s)
        return (long long)((k > l ? k - l : l - k) + 1) * p2 <= s;
    const long long stride = (p2 + s - 1) / s;
    return delta % stride == 0 && k == l;
}

// Block predicate of TRA_GRAN_BLOCK_EQ4 (radial, s a multiple of 128).
__device__ inline bool block_eq4_keep(const MaskDesc &m, int qb, int kb)
{
    const int sb = m.s / kBlock;
    return kb / sb < m.sink_frames || radial_keep(sb, qb, kb);
}

// Calls fn(lo, hi) for every kept run of keys of query q, cut to [a, b)
// and non-empty.  Runs never overlap.
template <class Fn>
__device__ void for_each_run(const MaskDesc &m, int q, int a, int b, Fn &&fn)
{
    auto emit = [&](int lo, int hi) {
        lo = imax(lo, a);
        hi = imin(hi, b);
        if (lo < hi)
            fn(lo, hi);
    };
    // Sink frames first; the family's runs then start past them.
    if (m.sink_frames > 0) {
        const long long sink_end = (long long)m.sink_frames * m.s;
        const int end = sink_end < m.n ? (int)sink_end : m.n;
        emit(0, end);
        a = imax(a, end);
        if (a >= b)
            return;
    }
    switch (m.kind) {
    case TRA_MASK_DENSE:
        emit(a, b);
        break;
    case TRA_MASK_SWA_CAUSAL: {
        const int i = q / m.s;
        emit(imax(0, i - m.window + 1) * m.s, (i + 1) * m.s);
        break;
    }
    case TRA_MASK_RADIAL: {
        const int s = m.s;
        const int i = q / s, k = q - i * s;
        const int j1 = (b - 1) / s;
        for (int j = a / s; j <= j1; ++j) {
            const int delta = i > j ? i - j : j - i;
            const int r = 31 - __clz(delta > 1 ? delta : 1);
            const long long p2 = 1ll << r;
            int lo, hi;
            if (p2 <= s) {
                const int w = s >> r;  // floor(s / 2^r) >= 1
                lo = imax(0, k - (w - 1));
                hi = imin(s - 1, k + (w - 1));
            } else {
                const long long stride = (p2 + s - 1) / s;  // ceil(2^r / s)
                if (delta % stride != 0)
                    continue;
                lo = hi = k;
            }
            emit(j * s + lo, j * s + hi + 1);
        }
        break;
    }
    case TRA_MASK_RADIUS3D: {
        const int hw = m.grid_h * m.grid_w;
        const int t = q / hw, rem = q - t * hw;
        const int h = rem / m.grid_w, w = rem - h * m.grid_w;
        const int t0 = imax(t - m.r_t, a / hw), t1 = imin(t + m.r_t, (b - 1) / hw);
        const int h0 = imax(0, h - m.r_s), h1 = imin(m.grid_h - 1, h + m.r_s);
        const int w0 = imax(0, w - m.r_s), w1 = imin(m.grid_w - 1, w + m.r_s);
        for (int tk = t0; tk <= t1; ++tk)
            for (int hk = h0; hk <= h1; ++hk) {
                const int base = tk * hw + hk * m.grid_w;
                emit(base + w0, base + w1 + 1);
            }
        break;
    }
    default:
        break;
    }
}

// Sum over the 128 threads of a workgroup (2 waves).
__device__ int block_sum_128(int v, int *scratch)
{
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0)
        scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    int tot = scratch[0] + scratch[1];
    __syncthreads();
    return tot;
}

// One workgroup of 128 threads per block; thread = query row of the block.
__global__ __launch_bounds__(128) void k_classify(MaskDesc m, int nkb, uint8_t *cls, int32_t *cnt)
{
    __shared__ int scratch[2];
    const long long id = blockIdx.x;
    const int qb = (int)(id / nkb), kb = (int)(id - (long long)qb * nkb);
    const int q = qb * kBlock + (int)threadIdx.x;
    const int a = kb * kBlock, b = imin(m.n, a + kBlock);
    int c = 0;
    if (q < m.n)
        for_each_run(m, q, a, b, [&](int lo, int hi) { c += hi - lo; });
    const int total = block_sum_128(c, scratch);
    if (threadIdx.x == 0) {
        const int rows_in = imin(kBlock, m.n - qb * kBlock);
        const int cols_in = b - a;
        uint8_t k;
        if (m.granularity == TRA_GRAN_BLOCK_EQ4)
            k = block_eq4_keep(m, qb, kb) ? kFull : kEmpty;  // n is a multiple of 128 here
        else if (total == 0)
            k = kEmpty;
        else if (cols_in < kBlock)
            k = kPartial;  // keys past n must be masked
        else if (m.granularity != TRA_GRAN_ELEMENT || total == rows_in * cols_in)
            k = kFull;
        else
            k = kPartial;
        cls[id] = k;
        cnt[id] = total;
    }
}

// One workgroup of 256 threads per block row: kept and partial block counts,
// predicate element count, attended element count.
__global__ __launch_bounds__(256) void k_row_stats(MaskDesc m, int nkb, const uint8_t *cls,
                                                   const int32_t *cnt, int32_t *row_blocks,
                                                   int32_t *row_partial, long long *row_pred,
                                                   long long *row_eff)
{
    __shared__ long long red[4][4];
    const int qb = blockIdx.x;
    const int rows_in = imin(kBlock, m.n - qb * kBlock);
    long long nb = 0, np = 0, pred = 0, eff = 0;
    for (int kb = threadIdx.x; kb < nkb; kb += 256) {
        const long long id = (long long)qb * nkb + kb;
        const uint8_t k = cls[id];
        pred += cnt[id];
        if (k != kEmpty) {
            nb++;
            np += (k == kPartial);
            const int cols_in = imin(kBlock, m.n - kb * kBlock);
            eff += (m.granularity == TRA_GRAN_ELEMENT) ? (long long)cnt[id]
                                                       : (long long)rows_in * cols_in;
        }
    }
    long long v[4] = {nb, np, pred, eff};
    for (int x = 0; x < 4; ++x)
        for (int off = 32; off > 0; off >>= 1)
            v[x] += __shfl_xor(v[x], off);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        for (int x = 0; x < 4; ++x)
            red[wave][x] = v[x];
    __syncthreads();
    if (threadIdx.x == 0) {
        long long t[4] = {0, 0, 0, 0};
        for (int w = 0; w < 4; ++w)
            for (int x = 0; x < 4; ++x)
                t[x] += red[w][x];
        row_blocks[qb] = (int32_t)t[0];
        row_partial[qb] = (int32_t)t[1];
        row_pred[qb] = t[2];
        row_eff[qb] = t[3];
    }
}

// One workgroup of 256 threads per block row: ascending CSR columns and the
// bitmask index of every partial block (numbered in CSR order).
__global__ __launch_bounds__(256) void k_compact(int nkb, const uint8_t *cls, const int32_t *row_ptr,
                                                 const int32_t *part_ptr, int32_t *col_idx,
                                                 int32_t *emask_idx, int32_t *part_list)
{
    __shared__ int wk[4], wp[4];
    const int qb = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int base_k = row_ptr[qb], base_p = part_ptr[qb];
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int kb0 = 0; kb0 < nkb; kb0 += 256) {
        const int kb = kb0 + (int)threadIdx.x;
        const uint8_t k = kb < nkb ? cls[(long long)qb * nkb + kb] : kEmpty;
        const unsigned long long bk = __ballot(k != kEmpty);
        const unsigned long long bp = __ballot(k == kPartial);
        if (lane == 0) {
            wk[wave] = __popcll(bk);
            wp[wave] = __popcll(bp);
        }
        __syncthreads();
        int ok = base_k, op = base_p;
        for (int w = 0; w < wave; ++w) {
            ok += wk[w];
            op += wp[w];
        }
        ok += __popcll(bk & below);
        op += __popcll(bp & below);
        if (k != kEmpty) {
            col_idx[ok] = kb;
            if (k == kPartial) {
                emask_idx[ok] = op;
                part_list[op] = qb * nkb + kb;
            } else {
                emask_idx[ok] = -1;
            }
        }
        for (int w = 0; w < 4; ++w) {
            base_k += wk[w];
            base_p += wp[w];
        }
        __syncthreads();
    }
}

// One workgroup of 128 threads per partial block; thread = row of the block.
__global__ __launch_bounds__(128) void k_fill_emask(MaskDesc m, int nkb, const int32_t *part_list,
                                                    uint32_t *emask)
{
    const int pi = blockIdx.x;
    const int id = part_list[pi];
    const int qb = id / nkb, kb = id - qb * nkb;
    const int r = threadIdx.x;
    const int q = qb * kBlock + r;
    const int a = kb * kBlock, b = imin(m.n, a + kBlock);
    uint32_t bits[4] = {0u, 0u, 0u, 0u};
    auto set_run = [&](int lo, int hi) {
        for (int x = lo - a; x < hi - a;) {
            const int w = x >> 5, bit = x & 31;
            const int len = imin(32 - bit, (hi - a) - x);
            const uint32_t run = (len == 32) ? 0xffffffffu : (((1u << len) - 1u) << bit);
            bits[w] |= run;
            x += len;
        }
    };
    if (q < m.n) {
        if (m.granularity == TRA_GRAN_ELEMENT)
            for_each_run(m, q, a, b, set_run);
        else
            set_run(a, b);  // whole block kept; only keys past n are dropped
    }
    uint4 out = make_uint4(bits[0], bits[1], bits[2], bits[3]);
    reinterpret_cast<uint4 *>(emask)[(size_t)pi * kBlock + r] = out;
}

__global__ void k_bitmap(int nqb, int nkb, int words, const uint8_t *cls, uint32_t *bitmap)
{
    const long long total = (long long)nqb * words;
    for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < total;
         x += (long long)gridDim.x * blockDim.x) {
        const int qb = (int)(x / words), w = (int)(x - (long long)qb * words);
        uint32_t v = 0;
        for (int bit = 0; bit < 32; ++bit) {
            const int kb = w * 32 + bit;
            if (kb < nkb && cls[(long long)qb * nkb + kb] != kEmpty)
                v |= 1u << bit;
        }
        bitmap[x] = v;
    }
}

}  // namespace

hipError_t launch_classify(const MaskDesc &m, int nqb, int nkb, uint8_t *cls, int32_t *cnt,
                           hipStream_t st)
{
    const long long blocks = (long long)nqb * nkb;
    hipLaunchKernelGGL(k_classify, dim3((unsigned)blocks), dim3(128), 0, st, m, nkb, cls, cnt);
    return hipGetLastError();
}

hipError_t launch_row_stats(const MaskDesc &m, int nqb, int nkb, const uint8_t *cls,
                            const int32_t *cnt, int32_t *row_blocks, int32_t *row_partial,
                            long long *row_pred, long long *row_eff, hipStream_t st)
{
    hipLaunchKernelGGL(k_row_stats, dim3(nqb), dim3(256), 0, st, m, nkb, cls, cnt, row_blocks,
                       row_partial, row_pred, row_eff);
    return hipGetLastError();
}

hipError_t launch_compact(int nqb, int nkb, const uint8_t *cls, const int32_t *row_ptr,
                          const int32_t *part_ptr, int32_t *col_idx, int32_t *emask_idx,
                          int32_t *part_list, hipStream_t st)
{
    hipLaunchKernelGGL(k_compact, dim3(nqb), dim3(256), 0, st, nkb, cls, row_ptr, part_ptr, col_idx,
                       emask_idx, part_list);
    return hipGetLastError();
}

hipError_t launch_fill_emask(const MaskDesc &m, int npartial, const int32_t *part_list, int nkb,
                             uint32_t *emask, hipStream_t st)
{
    if (npartial == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_fill_emask, dim3(npartial), dim3(128), 0, st, m, nkb, part_list, emask);
    return hipGetLastError();
}

hipError_t launch_bitmap(int nqb, int nkb, int words, const uint8_t *cls, uint32_t *bitmap,
                         hipStream_t st)
{
    const long long total = (long long)nqb * words;
    const long long want = (total + 255) / 256;
    const unsigned grid = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
    hipLaunchKernelGGL(k_bitmap, dim3(grid), dim3(256), 0, st, nqb, nkb, words, cls, bitmap);
    return hipGetLastError();
}

}  // namespace tra

// C ABI of libtra.so: argument checking, mask compilation driver, attention
// dispatch.  See include/tra.h for the contract of every entry point.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "probe.h"
#include "salad.h"
#include "tra_debug.h"
#include "tra_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

tra_status hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return TRA_OK;
    g_last_hip_error = (int32_t)e;
    return e == hipErrorOutOfMemory ? TRA_ERR_OOM : TRA_ERR_HIP;
}

#define TRA_HIP(expr)                              \
    do {                                           \
        const hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) {                    \
            st_ = hip_status(e_);                  \
            goto fail;                             \
        }                                          \
    } while (0)

// Every device buffer the library owns is allocated by dev_alloc and
// released by dev_free, which count the live ones.  A test can make the
// allocations fail from a given point on (tra_debug_fail_allocations) to run
// the error paths.
std::atomic<int64_t> g_live_allocs{0};
std::atomic<int64_t> g_fail_after{-1};

template <class T>
hipError_t dev_alloc(T **p, size_t count)
{
    *p = nullptr;
    for (int64_t left = g_fail_after.load(); left >= 0;) {
        if (left == 0)
            return hipErrorOutOfMemory;
        if (g_fail_after.compare_exchange_weak(left, left - 1))
            break;
    }
    const hipError_t e = hipMalloc((void **)p, std::max<size_t>(count, 1) * sizeof(T));
    if (e == hipSuccess)
        ++g_live_allocs;
    else
        *p = nullptr;
    return e;
}

void dev_free(void *p)
{
    if (p != nullptr && hipFree(p) == hipSuccess)
        --g_live_allocs;
}

using tra::PairSchedule;

void free_mask_buffers(tra_mask *m)
{
    dev_free(m->bitmap);
    dev_free(m->row_ptr);
    dev_free(m->col_idx);
    dev_free(m->emask_idx);
    dev_free(m->emask);
    dev_free(m->order);
    dev_free(m->pair_rows);
    dev_free(m->pair_ptr);
    dev_free(m->u_col);
    dev_free(m->u_em);
    dev_free(m->pair_order);
    dev_free(m->queue);
    dev_free(m->split_ctr);
    dev_free(m->split_ws);
    dev_free(m->t_pair_cols);
    dev_free(m->t_pair_ptr);
    dev_free(m->t_u_row);
    dev_free(m->t_u_em);
    dev_free(m->t_pair_order);
}

bool tensor_ok(const tra_tensor *t) { return t != nullptr && t->data != nullptr; }

// Kernel arguments shared by the forward and backward entry points (O and
// LSE may be NULL).
void fill_attn_args(tra::AttnArgs &a, const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V,
                    const tra_tensor *O, float *LSE, const tra_mask *mask, float scale)
{
    a.q = Q->data;
    a.k = K->data;
    a.v = V->data;
    a.o = O ? O->data : nullptr;
    a.lse = LSE;
    for (int i = 0; i < 3; ++i) {
        a.sq[i] = Q->stride[i];
        a.sk[i] = K->stride[i];
        a.sv[i] = V->stride[i];
        a.so[i] = O ? O->stride[i] : 0;
    }
    a.B = (int32_t)Q->B;
    a.H = (int32_t)Q->H;
    a.N = (int32_t)Q->N;
    a.D = (int32_t)Q->D;
    const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)Q->D);
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    a.mask.row_ptr = mask->row_ptr;
    a.mask.col_idx = mask->col_idx;
    a.mask.emask_idx = mask->emask_idx;
    a.mask.emask = mask->emask;
    a.mask.order = mask->order;
    a.mask.pair_rows = mask->pair_rows;
    a.mask.pair_ptr = mask->pair_ptr;
    a.mask.u_col = mask->u_col;
    a.mask.u_em = mask->u_em;
    a.mask.pair_order = mask->pair_order;
    a.mask.queue = mask->queue;
    a.mask.split_ctr = mask->split_ctr;
    a.mask.split_ws = mask->split_ws;
    a.mask.nqb = (int32_t)mask->info.nqb;
    a.mask.npairs = mask->npairs;
    a.mask.t_pair_cols = mask->t_pair_cols;
    a.mask.t_pair_ptr = mask->t_pair_ptr;
    a.mask.t_u_row = mask->t_u_row;
    a.mask.t_u_em = mask->t_u_em;
    a.mask.t_pair_order = mask->t_pair_order;
    a.mask.t_npairs = mask->t_npairs;
    a.Nk = a.N;
    a.part_o = nullptr;
    a.part_lse = nullptr;
    a.nsplit = a.split_tiles = a.nkv_tiles = a.stream_pairs = 0;
    a.tail_split = 0;
    a.split_min = 8;
    a.max_pair_tiles = mask->max_pair_tiles;
}

}  // namespace

namespace tra {

hipError_t resident_workgroups(const void *kern, int threads, long long *out)
{
    struct Entry {
        const void *kern;
        int dev, threads;
        long long grid;
    };
    static std::mutex mu;
    static std::vector<Entry> table;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : table)
            if (e.kern == kern && e.dev == dev && e.threads == threads) {
                *out = e.grid;
                return hipSuccess;
            }
    }
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
    if (err != hipSuccess)
        return err;
    const long long grid = (long long)cus * (per_cu < 1 ? 1 : per_cu);
    std::lock_guard<std::mutex> lock(mu);
    table.push_back({kern, dev, threads, grid});
    *out = grid;
    return hipSuccess;
}

}  // namespace tra

// Frame-streaming K/V cache (see tra_kvcache_create).
struct tra_kvcache {
    int64_t B, H, s, D;
    int32_t window;
    int device;
    int64_t appended;  // frames appended since creation or reset
    int32_t nsplit_max;
    int32_t cus;  // compute units of the device (queried at create)
    __bf16 *ring_k, *ring_v;  // [B, H, window * s, D]
    float *part_o, *part_lse;
};

extern "C" {

const char *tra_status_string(tra_status s)
{
    switch (s) {
    case TRA_OK:
        return "TRA_OK";
    case TRA_ERR_INVALID:
        return "TRA_ERR_INVALID";
    case TRA_ERR_UNSUPPORTED:
        return "TRA_ERR_UNSUPPORTED";
    case TRA_ERR_SHAPE:
        return "TRA_ERR_SHAPE";
    case TRA_ERR_OOM:
        return "TRA_ERR_OOM";
    case TRA_ERR_HIP:
        return "TRA_ERR_HIP";
    }
    return "TRA_ERR_UNKNOWN";
}

int32_t tra_last_hip_error(void) { return g_last_hip_error; }

int64_t tra_debug_live_allocations(void) { return g_live_allocs.load(); }

int64_t tra_debug_fail_allocations(int64_t after) { return g_fail_after.exchange(after < 0 ? -1 : after); }

int32_t tra_version(void) { return 100; /* 0.1.0 */ }

tra_status tra_probe_mfma_peak(int64_t iterations, int32_t blocks, float *out, int64_t *flops, void *hip_stream)
{
    if (iterations < 1 || blocks < 1 || out == nullptr || flops == nullptr)
        return TRA_ERR_INVALID;
    *flops = tra::mfma_loop_flops(iterations, blocks);
    return hip_status(tra::launch_mfma_loop(iterations, blocks, out, (hipStream_t)hip_stream));
}

tra_status tra_build_mask(int64_t f, int64_t s, int32_t kind, const tra_mask_params *p,
                          void *hip_stream, tra_mask **out)
{
    if (out == nullptr || p == nullptr)
        return TRA_ERR_INVALID;
    *out = nullptr;
    if (f < 1 || s < 1)
        return TRA_ERR_INVALID;
    if (kind < TRA_MASK_DENSE || kind > TRA_MASK_SWA_CAUSAL)
        return TRA_ERR_INVALID;
    if (p->granularity != TRA_GRAN_ELEMENT && p->granularity != TRA_GRAN_BLOCK_ANY &&
        p->granularity != TRA_GRAN_BLOCK_EQ4)
        return TRA_ERR_INVALID;
    for (int i = 0; i < 8; ++i)
        if (p->reserved[i] != 0)
            return TRA_ERR_INVALID;
    if (p->sink_frames < 0)
        return TRA_ERR_INVALID;
    if (p->granularity == TRA_GRAN_BLOCK_EQ4) {
        if (kind != TRA_MASK_RADIAL)
            return TRA_ERR_INVALID;
        if (s % tra::kBlock != 0)
            return TRA_ERR_UNSUPPORTED;
    }
    if (p->block != 0 && p->block != tra::kBlock)
        return TRA_ERR_UNSUPPORTED;
    const bool radius = kind == TRA_MASK_RADIUS3D, swa = kind == TRA_MASK_SWA_CAUSAL;
    if (!radius && (p->grid_h || p->grid_w || p->r_t || p->r_s))
        return TRA_ERR_INVALID;
    if (!swa && p->window)
        return TRA_ERR_INVALID;
    if (radius) {
        if (p->grid_h < 1 || p->grid_w < 1 || p->r_t < 0 || p->r_s < 0)
            return TRA_ERR_INVALID;
        if ((int64_t)p->grid_h * p->grid_w != s)
            return TRA_ERR_SHAPE;
    }
    if (swa && p->window < 1)
        return TRA_ERR_INVALID;
    if (f > INT32_MAX || s > INT32_MAX || f * s >= ((int64_t)1 << 31))
        return TRA_ERR_UNSUPPORTED;
    const int64_t n = f * s;
    const int64_t nb64 = (n + tra::kBlock - 1) / tra::kBlock;
    if (nb64 * nb64 >= ((int64_t)1 << 31))
        return TRA_ERR_UNSUPPORTED;  // block-class matrix indexed with 32 bits
    const int nqb = (int)nb64, nkb = (int)nb64;
    const int words = (nkb + 31) / 32;

    tra_mask *m = new (std::nothrow) tra_mask;
    if (m == nullptr)
        return TRA_ERR_OOM;
    std::memset(m, 0, sizeof(*m));
    tra::MaskDesc &d = m->desc;
    d.kind = kind;
    d.granularity = p->granularity;
    d.n = (int32_t)n;
    d.f = (int32_t)f;
    d.s = (int32_t)s;
    d.grid_h = p->grid_h;
    d.grid_w = p->grid_w;
    d.r_t = p->r_t;
    d.r_s = p->r_s;
    d.window = p->window;
    d.sink_frames = (int32_t)std::min<int64_t>(p->sink_frames, f);

    hipStream_t st = (hipStream_t)hip_stream;
    tra_status st_ = TRA_OK;
    uint8_t *cls = nullptr;
    int32_t *cnt = nullptr, *row_blocks = nullptr, *row_partial = nullptr, *part_ptr_d = nullptr,
            *part_list = nullptr;
    long long *row_pred = nullptr, *row_eff = nullptr;
    std::vector<int32_t> h_blocks(nqb), h_partial(nqb), h_row_ptr(nqb + 1), h_part_ptr(nqb + 1),
        h_order(nqb);
    std::vector<long long> h_pred(nqb), h_eff(nqb);
    std::vector<int32_t> h_col, h_em;
    PairSchedule ps, tps;
    int64_t nnz = 0, npart = 0;

    TRA_HIP(hipGetDevice(&m->device));
    TRA_HIP(dev_alloc(&cls, (size_t)nqb * nkb));
    TRA_HIP(dev_alloc(&cnt, (size_t)nqb * nkb));
    TRA_HIP(dev_alloc(&row_blocks, nqb));
    TRA_HIP(dev_alloc(&row_partial, nqb));
    TRA_HIP(dev_alloc(&row_pred, nqb));
    TRA_HIP(dev_alloc(&row_eff, nqb));
    TRA_HIP(tra::launch_classify(d, nqb, nkb, cls, cnt, st));
    TRA_HIP(tra::launch_row_stats(d, nqb, nkb, cls, cnt, row_blocks, row_partial, row_pred, row_eff, st));
    TRA_HIP(hipMemcpyAsync(h_blocks.data(), row_blocks, nqb * sizeof(int32_t), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipMemcpyAsync(h_partial.data(), row_partial, nqb * sizeof(int32_t), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipMemcpyAsync(h_pred.data(), row_pred, nqb * sizeof(long long), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipMemcpyAsync(h_eff.data(), row_eff, nqb * sizeof(long long), hipMemcpyDeviceToHost, st));
    TRA_HIP(hipStreamSynchronize(st));

    h_row_ptr[0] = 0;
    h_part_ptr[0] = 0;
    for (int r = 0; r < nqb; ++r) {
        nnz += h_blocks[r];
        npart += h_partial[r];
        if (nnz >= INT32_MAX) {
            st_ = TRA_ERR_UNSUPPORTED;
            goto fail;
        }
        h_row_ptr[r + 1] = (int32_t)nnz;
        h_part_ptr[r + 1] = (int32_t)npart;
    }
    // Within each chunk of kChunk consecutive query blocks, heaviest first.
    h_order = tra::chunk_order(std::vector<int64_t>(h_blocks.begin(), h_blocks.end()), tra::kChunk);

    TRA_HIP(dev_alloc(&m->row_ptr, nqb + 1));
    TRA_HIP(dev_alloc(&m->col_idx, (size_t)nnz));
    TRA_HIP(dev_alloc(&m->emask_idx, (size_t)nnz));
    TRA_HIP(dev_alloc(&m->emask, (size_t)npart * tra::kBlock * 4));
    TRA_HIP(dev_alloc(&m->order, nqb));
    TRA_HIP(dev_alloc(&m->bitmap, (size_t)nqb * words));
    TRA_HIP(dev_alloc(&m->queue, tra::kQueueWords));
    TRA_HIP(dev_alloc(&m->split_ctr, tra::kSplitSlots));
    TRA_HIP(dev_alloc(&m->split_ws, (size_t)2 * tra::kSplitSlots * tra::kSplitRecFloats));
    TRA_HIP(dev_alloc(&part_ptr_d, nqb + 1));
    TRA_HIP(dev_alloc(&part_list, (size_t)npart));
    TRA_HIP(hipMemcpyAsync(m->row_ptr, h_row_ptr.data(), (nqb + 1) * sizeof(int32_t), hipMemcpyHostToDevice, st));
    TRA_HIP(hipMemcpyAsync(part_ptr_d, h_part_ptr.data(), (nqb + 1) * sizeof(int32_t), hipMemcpyHostToDevice, st));
    TRA_HIP(hipMemcpyAsync(m->order, h_order.data(), nqb * sizeof(int32_t), hipMemcpyHostToDevice, st));
    TRA_HIP(hipMemsetAsync(m->queue, 0, tra::kQueueWords * sizeof(uint32_t), st));
    TRA_HIP(hipMemsetAsync(m->split_ctr, 0, tra::kSplitSlots * sizeof(uint32_t), st));
    TRA_HIP(tra::launch_compact(nqb, nkb, cls, m->row_ptr, part_ptr_d, m->col_idx, m->emask_idx, part_list, st));
    TRA_HIP(tra::launch_fill_emask(d, (int)npart, part_list, nkb, m->emask, st));
    TRA_HIP(tra::launch_bitmap(nqb, nkb, words, cls, m->bitmap, st));
    TRA_HIP(hipStreamSynchronize(st));

    // Pair schedule for the bf16 kernel, from the finished CSR.
    h_col.resize(nnz);
    h_em.resize(nnz);
    if (nnz) {
        TRA_HIP(hipMemcpy(h_col.data(), m->col_idx, nnz * sizeof(int32_t), hipMemcpyDeviceToHost));
        TRA_HIP(hipMemcpy(h_em.data(), m->emask_idx, nnz * sizeof(int32_t), hipMemcpyDeviceToHost));
    }
    ps = tra::build_pairs(nqb, s, h_row_ptr, h_col, h_em);
    m->npairs = (int32_t)(ps.rows.size() / 2);
    for (int32_t p = 0; p < m->npairs; ++p)
        m->max_pair_tiles = std::max(m->max_pair_tiles, ps.ptr[p + 1] - ps.ptr[p]);
    TRA_HIP(dev_alloc(&m->pair_rows, ps.rows.size()));
    TRA_HIP(dev_alloc(&m->pair_ptr, ps.ptr.size()));
    TRA_HIP(dev_alloc(&m->u_col, ps.col.size()));
    TRA_HIP(dev_alloc(&m->u_em, ps.em.size()));
    TRA_HIP(dev_alloc(&m->pair_order, ps.order.size()));
    TRA_HIP(hipMemcpy(m->pair_rows, ps.rows.data(), ps.rows.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    TRA_HIP(hipMemcpy(m->pair_ptr, ps.ptr.data(), ps.ptr.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    if (!ps.col.empty()) {
        TRA_HIP(hipMemcpy(m->u_col, ps.col.data(), ps.col.size() * sizeof(int32_t), hipMemcpyHostToDevice));
        TRA_HIP(hipMemcpy(m->u_em, ps.em.data(), ps.em.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    }
    TRA_HIP(hipMemcpy(m->pair_order, ps.order.data(), ps.order.size() * sizeof(int32_t), hipMemcpyHostToDevice));

    // The same schedule over key blocks, from the column lists of the mask.
    {
        std::vector<int32_t> col_ptr, row_idx, em_t;
        tra::transpose_csr(nqb, nkb, h_row_ptr, h_col, h_em, col_ptr, row_idx, em_t);
        tps = tra::build_pairs(nkb, s, col_ptr, row_idx, em_t);
    }
    m->t_npairs = (int32_t)(tps.rows.size() / 2);
    m->t_nunion = (int64_t)tps.col.size();
    TRA_HIP(dev_alloc(&m->t_pair_cols, tps.rows.size()));
    TRA_HIP(dev_alloc(&m->t_pair_ptr, tps.ptr.size()));
    TRA_HIP(dev_alloc(&m->t_u_row, tps.col.size()));
    TRA_HIP(dev_alloc(&m->t_u_em, tps.em.size()));
    TRA_HIP(dev_alloc(&m->t_pair_order, tps.order.size()));
    TRA_HIP(hipMemcpy(m->t_pair_cols, tps.rows.data(), tps.rows.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    TRA_HIP(hipMemcpy(m->t_pair_ptr, tps.ptr.data(), tps.ptr.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    if (!tps.col.empty()) {
        TRA_HIP(hipMemcpy(m->t_u_row, tps.col.data(), tps.col.size() * sizeof(int32_t), hipMemcpyHostToDevice));
        TRA_HIP(hipMemcpy(m->t_u_em, tps.em.data(), tps.em.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    }
    TRA_HIP(hipMemcpy(m->t_pair_order, tps.order.data(), tps.order.size() * sizeof(int32_t), hipMemcpyHostToDevice));

    {
        tra_mask_info &in = m->info;
        in.n = n;
        in.f = f;
        in.s = s;
        in.nqb = nqb;
        in.nkb = nkb;
        in.kept_blocks = nnz;
        in.partial_blocks = npart;
        in.pred_elems = 0;
        in.kept_elems = 0;
        for (int r = 0; r < nqb; ++r) {
            in.pred_elems += h_pred[r];
            in.kept_elems += h_eff[r];
        }
        in.min_row_blocks = *std::min_element(h_blocks.begin(), h_blocks.end());
        in.max_row_blocks = *std::max_element(h_blocks.begin(), h_blocks.end());
        in.bitmap_words = words;
        in.work_items = m->npairs;
        in.tile_loads = (int64_t)ps.col.size();
        in.kind = kind;
        in.granularity = p->granularity;
        in.bwd_work_items = m->t_npairs;
        in.bwd_tile_loads = m->t_nunion;
    }
    dev_free(cls);
    dev_free(cnt);
    dev_free(row_blocks);
    dev_free(row_partial);
    dev_free(row_pred);
    dev_free(row_eff);
    dev_free(part_ptr_d);
    dev_free(part_list);
    *out = m;
    return TRA_OK;

fail:
    (void)hipStreamSynchronize(st);
    dev_free(cls);
    dev_free(cnt);
    dev_free(row_blocks);
    dev_free(row_partial);
    dev_free(row_pred);
    dev_free(row_eff);
    dev_free(part_ptr_d);
    dev_free(part_list);
    free_mask_buffers(m);
    delete m;
    return st_;
}

tra_status tra_mask_get_info(const tra_mask *m, tra_mask_info *out)
{
    if (m == nullptr || out == nullptr)
        return TRA_ERR_INVALID;
    *out = m->info;
    return TRA_OK;
}

tra_status tra_mask_export(const tra_mask *m, uint32_t *bitmap, int32_t *row_ptr, int32_t *col_idx,
                           int32_t *emask_idx, uint32_t *emask, int32_t *order)
{
    if (m == nullptr)
        return TRA_ERR_INVALID;
    const tra_mask_info &in = m->info;
    tra_status st_ = TRA_OK;
    if (bitmap)
        TRA_HIP(hipMemcpy(bitmap, m->bitmap, (size_t)in.nqb * in.bitmap_words * sizeof(uint32_t), hipMemcpyDeviceToHost));
    if (row_ptr)
        TRA_HIP(hipMemcpy(row_ptr, m->row_ptr, (size_t)(in.nqb + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));
    if (col_idx && in.kept_blocks)
        TRA_HIP(hipMemcpy(col_idx, m->col_idx, (size_t)in.kept_blocks * sizeof(int32_t), hipMemcpyDeviceToHost));
    if (emask_idx && in.kept_blocks)
        TRA_HIP(hipMemcpy(emask_idx, m->emask_idx, (size_t)in.kept_blocks * sizeof(int32_t), hipMemcpyDeviceToHost));
    if (emask && in.partial_blocks)
        TRA_HIP(hipMemcpy(emask, m->emask, (size_t)in.partial_blocks * tra::kBlock * 4 * sizeof(uint32_t), hipMemcpyDeviceToHost));
    if (order)
        TRA_HIP(hipMemcpy(order, m->order, (size_t)in.nqb * sizeof(int32_t), hipMemcpyDeviceToHost));
    return TRA_OK;
fail:
    return st_;
}

void tra_mask_free(tra_mask *m)
{
    if (m == nullptr)
        return;
    free_mask_buffers(m);
    delete m;
}

tra_status tra_sparse_attn_fwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V,
                               const tra_mask *mask, tra_tensor *O, float *LSE, float scale,
                               void *hip_stream)
{
    if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr || mask == nullptr)
        return TRA_ERR_INVALID;
    const tra_tensor *ts[4] = {Q, K, V, O};
    const bool empty = Q->B == 0 || Q->H == 0;  // empty tensors may carry a NULL pointer
    if (!empty && (!tensor_ok(Q) || !tensor_ok(K) || !tensor_ok(V) || !tensor_ok(O)))
        return TRA_ERR_INVALID;
    for (const tra_tensor *t : ts) {
        if (t->B != Q->B || t->H != Q->H || t->N != Q->N || t->D != Q->D)
            return TRA_ERR_SHAPE;
        if (t->B < 0 || t->H < 0 || t->N < 0 || t->D < 0)
            return TRA_ERR_SHAPE;
    }
    if (Q->N != mask->info.n)
        return TRA_ERR_SHAPE;
    for (const tra_tensor *t : ts)
        if (t->dtype != Q->dtype)
            return TRA_ERR_UNSUPPORTED;
    if (Q->dtype != TRA_BF16 && Q->dtype != TRA_F32)
        return TRA_ERR_UNSUPPORTED;
    if (Q->D != 64 && Q->D != 128)
        return TRA_ERR_UNSUPPORTED;
    const int64_t vec = Q->dtype == TRA_BF16 ? 8 : 4;  // elements per 16-byte access
    for (const tra_tensor *t : ts) {
        if (t->stride[3] != 1)
            return TRA_ERR_UNSUPPORTED;
        for (int i = 0; i < 3; ++i)
            if (t->stride[i] < 0 || t->stride[i] % vec != 0)
                return TRA_ERR_UNSUPPORTED;
        if (((uintptr_t)t->data) % 16 != 0)
            return TRA_ERR_UNSUPPORTED;
    }
    if (empty)
        return TRA_OK;
    if (Q->B * Q->H * mask->info.nqb >= ((int64_t)1 << 31) || Q->B * Q->H * Q->N >= ((int64_t)1 << 40))
        return TRA_ERR_UNSUPPORTED;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev != mask->device)
        return TRA_ERR_INVALID;

    tra::AttnArgs a;
    fill_attn_args(a, Q, K, V, O, LSE, mask, scale);
    hipStream_t st = (hipStream_t)hip_stream;
    e = Q->dtype == TRA_BF16 ? tra::launch_attn_bf16(a, st) : tra::launch_attn_f32(a, st);
    return hip_status(e);
}

size_t tra_sparse_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D)
{
    if (B < 0 || H < 0 || N < 0 || (D != 64 && D != 128))
        return 0;
    return tra::bwd_workspace(B, H, N, D).bytes;
}

tra_status tra_sparse_attn_bwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V, const tra_tensor *O,
                               const tra_tensor *dO, const float *LSE, const tra_mask *mask, tra_tensor *dQ,
                               tra_tensor *dK, tra_tensor *dV, void *workspace, size_t workspace_bytes, float scale,
                               void *hip_stream)
{
    const tra_tensor *ts[9] = {Q, K, V, O, dO, dQ, dK, dV, nullptr};
    for (int i = 0; i < 8; ++i)
        if (ts[i] == nullptr)
            return TRA_ERR_INVALID;
    if (mask == nullptr)
        return TRA_ERR_INVALID;
    const bool empty = Q->B == 0 || Q->H == 0;
    if (!empty) {
        for (int i = 0; i < 8; ++i)
            if (!tensor_ok(ts[i]))
                return TRA_ERR_INVALID;
        if (LSE == nullptr || workspace == nullptr)
            return TRA_ERR_INVALID;
    }
    for (int i = 0; i < 8; ++i) {
        const tra_tensor *t = ts[i];
        if (t->B != Q->B || t->H != Q->H || t->N != Q->N || t->D != Q->D)
            return TRA_ERR_SHAPE;
        if (t->B < 0 || t->H < 0 || t->N < 0 || t->D < 0)
            return TRA_ERR_SHAPE;
    }
    if (Q->N != mask->info.n)
        return TRA_ERR_SHAPE;
    if (Q->dtype != TRA_BF16 && Q->dtype != TRA_F32)
        return TRA_ERR_UNSUPPORTED;
    for (int i = 0; i < 8; ++i)
        if (ts[i]->dtype != Q->dtype)
            return TRA_ERR_UNSUPPORTED;
    if (Q->D != 64 && Q->D != 128)
        return TRA_ERR_UNSUPPORTED;
    const int64_t vec = Q->dtype == TRA_BF16 ? 8 : 4;  // elements per 16 bytes
    for (int i = 0; i < 8; ++i) {
        const tra_tensor *t = ts[i];
        if (t->stride[3] != 1)
            return TRA_ERR_UNSUPPORTED;
        for (int j = 0; j < 3; ++j)
            if (t->stride[j] < 0 || t->stride[j] % vec != 0)
                return TRA_ERR_UNSUPPORTED;
        if (((uintptr_t)t->data) % 16 != 0)
            return TRA_ERR_UNSUPPORTED;
    }
    if (empty)
        return TRA_OK;
    if (Q->B * Q->H * mask->info.nqb >= ((int64_t)1 << 31) || Q->B * Q->H * Q->N >= ((int64_t)1 << 40))
        return TRA_ERR_UNSUPPORTED;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    if (dev != mask->device)
        return TRA_ERR_INVALID;

    const tra::BwdWorkspace ws = tra::bwd_workspace(Q->B, Q->H, Q->N, Q->D);
    if (workspace_bytes < ws.bytes || ((uintptr_t)workspace) % 256 != 0)
        return TRA_ERR_INVALID;

    tra::BwdArgs a;
    std::memset(&a, 0, sizeof(a));
    fill_attn_args(a.f, Q, K, V, nullptr, nullptr, mask, scale);
    a.o = O->data;
    a.dout = dO->data;
    a.dq = dQ->data;
    a.dk = dK->data;
    a.dv = dV->data;
    a.lse = LSE;
    a.delta = (float *)((char *)workspace + ws.delta);
    a.nlse = (float *)((char *)workspace + ws.nlse);
    for (int i = 0; i < 3; ++i) {
        a.s_o[i] = O->stride[i];
        a.s_do[i] = dO->stride[i];
        a.s_dq[i] = dQ->stride[i];
        a.s_dk[i] = dK->stride[i];
        a.s_dv[i] = dV->stride[i];
    }
    return hip_status(Q->dtype == TRA_BF16 ? tra::launch_attn_bwd_bf16(a, (hipStream_t)hip_stream)
                                           : tra::launch_attn_bwd_f32(a, (hipStream_t)hip_stream));
}

tra_status tra_kvcache_create(int64_t B, int64_t H, int64_t s, int64_t D, int32_t window, int32_t dtype,
                              tra_kvcache **out)
{
    if (out == nullptr)
        return TRA_ERR_INVALID;
    *out = nullptr;
    if (B < 1 || H < 1 || s < 1 || window < 1)
        return TRA_ERR_INVALID;
    if (dtype != TRA_BF16 || (D != 64 && D != 128) || s % tra::kBlock != 0)
        return TRA_ERR_UNSUPPORTED;
    const int64_t ring_rows = (int64_t)window * s;
    if (ring_rows >= ((int64_t)1 << 31) || B * H * ring_rows >= ((int64_t)1 << 40))
        return TRA_ERR_UNSUPPORTED;
    tra_kvcache *c = new (std::nothrow) tra_kvcache;
    if (c == nullptr)
        return TRA_ERR_OOM;
    std::memset(c, 0, sizeof(*c));
    c->B = B;
    c->H = H;
    c->s = s;
    c->D = D;
    c->window = window;
    c->nsplit_max = (int32_t)(ring_rows / tra::kBlock);
    const size_t ring = (size_t)(B * H * ring_rows * D);
    const size_t rows = (size_t)(B * H * s);
    tra_status st_ = TRA_OK;
    TRA_HIP(hipGetDevice(&c->device));
    TRA_HIP(hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, c->device));
    TRA_HIP(dev_alloc(&c->ring_k, ring));
    TRA_HIP(dev_alloc(&c->ring_v, ring));
    TRA_HIP(dev_alloc(&c->part_o, (size_t)c->nsplit_max * rows * D));
    TRA_HIP(dev_alloc(&c->part_lse, (size_t)c->nsplit_max * rows));
    *out = c;
    return TRA_OK;
fail:
    dev_free(c->ring_k);
    dev_free(c->ring_v);
    dev_free(c->part_o);
    dev_free(c->part_lse);
    delete c;
    return st_;
}

static tra_status check_frame_tensor(const tra_kvcache *c, const tra_tensor *t)
{
    if (t == nullptr || t->data == nullptr)
        return TRA_ERR_INVALID;
    if (t->B != c->B || t->H != c->H || t->N != c->s || t->D != c->D)
        return TRA_ERR_SHAPE;
    if (t->dtype != TRA_BF16)
        return TRA_ERR_UNSUPPORTED;
    if (t->stride[3] != 1)
        return TRA_ERR_UNSUPPORTED;
    for (int j = 0; j < 3; ++j)
        if (t->stride[j] < 0 || t->stride[j] % 8 != 0)
            return TRA_ERR_UNSUPPORTED;
    if (((uintptr_t)t->data) % 16 != 0)
        return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

static tra_status check_device(const tra_kvcache *c)
{
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_status(e);
    return dev == c->device ? TRA_OK : TRA_ERR_INVALID;
}

tra_status tra_kvcache_append(tra_kvcache *c, const tra_tensor *K, const tra_tensor *V, void *hip_stream)
{
    if (c == nullptr)
        return TRA_ERR_INVALID;
    tra_status st = check_frame_tensor(c, K);
    if (st == TRA_OK)
        st = check_frame_tensor(c, V);
    if (st == TRA_OK)
        st = check_device(c);
    if (st != TRA_OK)
        return st;
    const int64_t ring_rows = (int64_t)c->window * c->s;
    const int64_t row0 = (c->appended % c->window) * c->s;
    hipStream_t hs = (hipStream_t)hip_stream;
    const hipError_t e = tra::launch_ring_copy(K->data, K->stride, c->ring_k, V->data, V->stride, c->ring_v, c->B,
                                               c->H, c->s, c->D, ring_rows, row0, hs);
    if (e != hipSuccess)
        return hip_status(e);
    c->appended++;
    return TRA_OK;
}

tra_status tra_kvcache_attn(tra_kvcache *c, const tra_tensor *Q, tra_tensor *O, float *LSE, float scale,
                            void *hip_stream)
{
    if (c == nullptr)
        return TRA_ERR_INVALID;
    tra_status st = check_frame_tensor(c, Q);
    if (st == TRA_OK)
        st = check_frame_tensor(c, O);
    if (st == TRA_OK)
        st = check_device(c);
    if (st != TRA_OK)
        return st;
    if (c->appended == 0)
        return TRA_ERR_INVALID;
    const int64_t frames = std::min<int64_t>(c->appended, c->window);
    const int64_t ring_rows = (int64_t)c->window * c->s;

    tra::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = Q->data;
    a.k = c->ring_k;
    a.v = c->ring_v;
    a.o = O->data;
    a.lse = LSE;
    for (int i = 0; i < 3; ++i) {
        a.sq[i] = Q->stride[i];
        a.so[i] = O->stride[i];
    }
    a.sk[0] = a.sv[0] = c->H * ring_rows * c->D;
    a.sk[1] = a.sv[1] = ring_rows * c->D;
    a.sk[2] = a.sv[2] = c->D;
    a.B = (int32_t)c->B;
    a.H = (int32_t)c->H;
    a.N = (int32_t)c->s;
    a.Nk = (int32_t)ring_rows;
    a.D = (int32_t)c->D;
    const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)c->D);
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    a.mask.nqb = (int32_t)(c->s / tra::kBlock);
    a.stream_pairs = (a.mask.nqb + 1) / 2;
    a.nkv_tiles = (int32_t)(frames * c->s / tra::kBlock);
    // about one workgroup per two compute units: more splits cost more in
    // partial outputs and merging than they gain in parallelism (measured at
    // 16 heads x 256 tokens x 16 frames: 41.7 us with 512 workgroups, 25.0 us
    // with 128, 28.1 us with 64)
    const int cus = c->cus > 0 ? c->cus : 256;
    const int64_t base = c->B * c->H * a.stream_pairs;
    int64_t want = ((int64_t)cus / 2 + base - 1) / base;
    want = std::max<int64_t>(1, std::min<int64_t>(want, a.nkv_tiles));
    a.split_tiles = (int32_t)((a.nkv_tiles + want - 1) / want);
    a.nsplit = (a.nkv_tiles + a.split_tiles - 1) / a.split_tiles;
    a.part_o = c->part_o;
    a.part_lse = c->part_lse;
    return hip_status(tra::launch_attn_stream_bf16(a, (hipStream_t)hip_stream));
}

tra_status tra_kvcache_get_frames(const tra_kvcache *c, int64_t *appended, int64_t *cached)
{
    if (c == nullptr)
        return TRA_ERR_INVALID;
    if (appended)
        *appended = c->appended;
    if (cached)
        *cached = std::min<int64_t>(c->appended, c->window);
    return TRA_OK;
}

tra_status tra_kvcache_reset(tra_kvcache *c)
{
    if (c == nullptr)
        return TRA_ERR_INVALID;
    c->appended = 0;
    return TRA_OK;
}

void tra_kvcache_free(tra_kvcache *c)
{
    if (c == nullptr)
        return;
    dev_free(c->ring_k);
    dev_free(c->ring_v);
    dev_free(c->part_o);
    dev_free(c->part_lse);
    delete c;
}


size_t tra_linear_attn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D)
{
    if (B < 0 || H < 0 || N < 0 || (D != 64 && D != 128))
        return 0;
    return tra::linear_workspace_bytes(B, H, N, D);
}

tra_status tra_linear_attn_fwd(const tra_tensor *Q, const tra_tensor *K, const tra_tensor *V, tra_tensor *O,
                               float eps, void *workspace, size_t workspace_bytes, void *hip_stream)
{
    const tra_tensor *ts[4] = {Q, K, V, O};
    for (const tra_tensor *t : ts)
        if (t == nullptr)
            return TRA_ERR_INVALID;
    const bool empty = Q->B == 0 || Q->H == 0 || Q->N == 0;
    for (const tra_tensor *t : ts) {
        if (t->B != Q->B || t->H != Q->H || t->N != Q->N || t->D != Q->D)
            return TRA_ERR_SHAPE;
        if (t->B < 0 || t->H < 0 || t->N < 0 || t->D < 0)
            return TRA_ERR_SHAPE;
    }
    for (const tra_tensor *t : ts)
        if (t->dtype != TRA_BF16)
            return TRA_ERR_UNSUPPORTED;
    if (Q->D != 64 && Q->D != 128)
        return TRA_ERR_UNSUPPORTED;
    if (!(eps >= 0.f))
        return TRA_ERR_INVALID;
    for (const tra_tensor *t : ts) {
        if (t->stride[3] != 1)
            return TRA_ERR_UNSUPPORTED;
        for (int j = 0; j < 3; ++j)
            if (t->stride[j] < 0 || t->stride[j] % 8 != 0)
                return TRA_ERR_UNSUPPORTED;
    }
    if (empty)
        return TRA_OK;
    for (const tra_tensor *t : ts)
        if (t->data == nullptr || ((uintptr_t)t->data) % 16 != 0)
            return t->data == nullptr ? TRA_ERR_INVALID : TRA_ERR_UNSUPPORTED;
    if (Q->N >= ((int64_t)1 << 31) || Q->B * Q->H * Q->N >= ((int64_t)1 << 40))
        return TRA_ERR_UNSUPPORTED;
    if (workspace == nullptr || workspace_bytes < tra::linear_workspace_bytes(Q->B, Q->H, Q->N, Q->D) ||
        ((uintptr_t)workspace) % 256 != 0)
        return TRA_ERR_INVALID;
    return hip_status(tra::launch_linear_attn_bf16(Q->data, Q->stride, K->data, K->stride, V->data, V->stride,
                                                   O->data, O->stride, Q->B, Q->H, Q->N, Q->D, eps, workspace,
                                                   (hipStream_t)hip_stream));
}

size_t tra_salad_gate_workspace_bytes(int64_t B, int64_t N)
{
    if (B < 0 || N < 0)
        return 0;
    return tra::salad_gate_workspace_bytes(B, N);
}

// Checks shared by the two gate entry points (all but the workspace).
static tra_status check_gate_args(const tra_tensor *X, const void *w, const float *gate)
{
    if (X == nullptr)
        return TRA_ERR_INVALID;
    if (X->B < 0 || X->N < 0 || X->D < 0 || X->H != 1)
        return TRA_ERR_SHAPE;
    if (X->dtype != TRA_BF16)
        return TRA_ERR_UNSUPPORTED;
    const int64_t C = X->D;
    if (C == 0 || C % 8 != 0 || C > 8192)
        return TRA_ERR_UNSUPPORTED;
    if (X->stride[3] != 1 || X->stride[0] < 0 || X->stride[0] % 8 != 0 || X->stride[2] < 0 ||
        X->stride[2] % 8 != 0)
        return TRA_ERR_UNSUPPORTED;
    if (X->B == 0)
        return TRA_OK;
    if (X->N == 0)
        return TRA_ERR_INVALID;  // the mean over no tokens is undefined
    if (X->data == nullptr || w == nullptr || gate == nullptr)
        return TRA_ERR_INVALID;
    if (((uintptr_t)X->data) % 16 != 0 || ((uintptr_t)w) % 16 != 0)
        return TRA_ERR_UNSUPPORTED;
    if (X->B >= 65536 || X->N >= ((int64_t)1 << 40))
        return TRA_ERR_UNSUPPORTED;
    return TRA_OK;
}

tra_status tra_salad_gate(const tra_tensor *X, const void *w, float bias, float *gate, void *workspace,
                          size_t workspace_bytes, void *hip_stream)
{
    const tra_status st = check_gate_args(X, w, gate);
    if (st != TRA_OK || X->B == 0)
        return st;
    if (workspace == nullptr || workspace_bytes < tra::salad_gate_workspace_bytes(X->B, X->N) ||
        ((uintptr_t)workspace) % 256 != 0)
        return TRA_ERR_INVALID;
    const int64_t sx[2] = {X->stride[0], X->stride[2]};
    return hip_status(tra::launch_salad_gate(X->data, sx, w, bias, X->B, X->N, X->D, gate, workspace,
                                             (hipStream_t)hip_stream));
}

tra_status tra_salad_gate_noalloc(const tra_tensor *X, const void *w, float bias, float *gate, void *hip_stream)
{
    const tra_status st = check_gate_args(X, w, gate);
    if (st != TRA_OK || X->B == 0)
        return st;
    if (!tra::salad_gate_scratch_fits(X->B, X->N))
        return TRA_ERR_UNSUPPORTED;
    const int64_t sx[2] = {X->stride[0], X->stride[2]};
    return hip_status(tra::launch_salad_gate_scratch(X->data, sx, w, bias, X->B, X->N, X->D, gate,
                                                     (hipStream_t)hip_stream));
}

tra_status tra_salad_combine(const tra_tensor *O_sparse, const tra_tensor *O_lin, const void *W, const float *bias,
                             const float *gate, tra_tensor *out, void *hip_stream)
{
    const tra_tensor *ts[3] = {O_sparse, O_lin, out};
    for (const tra_tensor *t : ts)
        if (t == nullptr)
            return TRA_ERR_INVALID;
    for (const tra_tensor *t : ts) {
        if (t->B != O_sparse->B || t->H != O_sparse->H || t->N != O_sparse->N || t->D != O_sparse->D)
            return TRA_ERR_SHAPE;
        if (t->B < 0 || t->H < 0 || t->N < 0 || t->D < 0)
            return TRA_ERR_SHAPE;
    }
    for (const tra_tensor *t : ts)
        if (t->dtype != TRA_BF16)
            return TRA_ERR_UNSUPPORTED;
    const int64_t B = O_sparse->B, H = O_sparse->H, N = O_sparse->N, D = O_sparse->D;
    if (D != 64 && D != 128)
        return TRA_ERR_UNSUPPORTED;
    for (const tra_tensor *t : ts) {
        if (t->stride[3] != 1)
            return TRA_ERR_UNSUPPORTED;
        for (int j = 0; j < 3; ++j)
            if (t->stride[j] < 0 || t->stride[j] % 8 != 0)
                return TRA_ERR_UNSUPPORTED;
    }
    const int64_t C = H * D;
    if (B == 0 || H == 0 || N == 0)
        return TRA_OK;
    if (C % 64 != 0 || C > 65536)
        return TRA_ERR_UNSUPPORTED;
    for (const tra_tensor *t : ts)
        if (t->data == nullptr)
            return TRA_ERR_INVALID;
    if (W == nullptr || gate == nullptr)
        return TRA_ERR_INVALID;
    if (out->data == O_lin->data)
        return TRA_ERR_INVALID;
    if (out->data == O_sparse->data)
        for (int j = 0; j < 3; ++j)
            if (out->stride[j] != O_sparse->stride[j])
                return TRA_ERR_INVALID;
    for (const tra_tensor *t : ts)
        if (((uintptr_t)t->data) % 16 != 0)
            return TRA_ERR_UNSUPPORTED;
    if (((uintptr_t)W) % 16 != 0 || (bias != nullptr && ((uintptr_t)bias) % 16 != 0))
        return TRA_ERR_UNSUPPORTED;
    if (B * N >= ((int64_t)1 << 31))
        return TRA_ERR_UNSUPPORTED;
    return hip_status(tra::launch_salad_combine(O_sparse->data, O_sparse->stride, O_lin->data, O_lin->stride,
                                                out->data, out->stride, W, bias, gate, B, H, N, D,
                                                (hipStream_t)hip_stream));
}

}  // extern "C"

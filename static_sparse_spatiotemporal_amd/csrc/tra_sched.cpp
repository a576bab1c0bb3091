// Host-side work schedules of a compiled mask (see tra_sched.h).
#include "tra_sched.h"

#include <stdint.h>

#include <algorithm>
#include <numeric>

namespace tra {

double jaccard(const int32_t *a, int na, const int32_t *b, int nb)
{
    int i = 0, j = 0, inter = 0;
    while (i < na && j < nb) {
        if (a[i] == b[j]) {
            ++inter;
            ++i;
            ++j;
        } else if (a[i] < b[j]) {
            ++i;
        } else {
            ++j;
        }
    }
    const int uni = na + nb - inter;
    return uni ? (double)inter / uni : 1.0;
}

std::vector<int32_t> chunk_order(const std::vector<int64_t> &weight, int chunk)
{
    const int n = (int)weight.size();
    std::vector<int32_t> order(n);
    std::iota(order.begin(), order.end(), 0);
    for (int c0 = 0; c0 < n; c0 += chunk)
        std::stable_sort(order.begin() + c0, order.begin() + std::min(n, c0 + chunk),
                         [&](int x, int y) { return weight[x] > weight[y]; });
    return order;
}

PairSchedule build_pairs(int nrows, int64_t s, const std::vector<int32_t> &ptr, const std::vector<int32_t> &col,
                         const std::vector<int32_t> &em)
{
    PairSchedule ps;
    std::vector<int> offs = {1};
    if (s % kBlock == 0 && s / kBlock > 1)
        offs.push_back((int)(s / kBlock));
    std::vector<char> used(nrows, 0);
    auto list = [&](int r) { return col.data() + ptr[r]; };
    auto len = [&](int r) { return ptr[r + 1] - ptr[r]; };
    for (int r = 0; r < nrows; ++r) {
        if (used[r])
            continue;
        int best = -1;
        double bj = 0.0;
        for (int off : offs) {
            const int r2 = r + off;
            if (r2 >= nrows || used[r2])
                continue;
            const double j = jaccard(list(r), len(r), list(r2), len(r2));
            if (j > bj) {
                bj = j;
                best = r2;
            }
        }
        used[r] = 1;
        if (best >= 0)
            used[best] = 1;
        ps.rows.push_back(r);
        ps.rows.push_back(best);
    }
    const int np = (int)ps.rows.size() / 2;
    ps.ptr.assign(np + 1, 0);
    std::vector<int64_t> weight(np);
    for (int p = 0; p < np; ++p) {
        const int a = ps.rows[2 * p], b = ps.rows[2 * p + 1];
        int i = ptr[a], ie = ptr[a + 1];
        int j = b >= 0 ? ptr[b] : 0, je = b >= 0 ? ptr[b + 1] : 0;
        while (i < ie || j < je) {
            const int ca = i < ie ? col[i] : INT32_MAX;
            const int cb = j < je ? col[j] : INT32_MAX;
            const int c = ca < cb ? ca : cb;
            ps.col.push_back(c);
            ps.em.push_back(ca == c ? em[i++] : kAbsent);
            ps.em.push_back(cb == c ? em[j++] : kAbsent);
        }
        ps.ptr[p + 1] = (int32_t)ps.col.size();
        weight[p] = ps.ptr[p + 1] - ps.ptr[p];
    }
    ps.order = chunk_order(weight, kPairChunk);
    return ps;
}

void transpose_csr(int nrows, int ncols, const std::vector<int32_t> &ptr, const std::vector<int32_t> &col,
                   const std::vector<int32_t> &em, std::vector<int32_t> &col_ptr, std::vector<int32_t> &row_idx,
                   std::vector<int32_t> &em_t)
{
    const int64_t nnz = ptr[nrows];
    col_ptr.assign(ncols + 1, 0);
    row_idx.assign(nnz, 0);
    em_t.assign(nnz, 0);
    for (int64_t e = 0; e < nnz; ++e)
        col_ptr[col[e] + 1]++;
    for (int c = 0; c < ncols; ++c)
        col_ptr[c + 1] += col_ptr[c];
    std::vector<int32_t> fill(col_ptr.begin(), col_ptr.end() - 1);
    for (int r = 0; r < nrows; ++r)  // rows in order: each column list ascends
        for (int32_t e = ptr[r]; e < ptr[r + 1]; ++e) {
            const int32_t at = fill[col[e]]++;
            row_idx[at] = r;
            em_t[at] = em[e];
        }
}

}  // namespace tra

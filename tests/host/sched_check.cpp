// Checks of the host-side schedule builders (tra_sched.cpp) on seeded random
// and banded block masks, meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Exit status 0 when every check holds; the
// first violation is printed and exits 1.
//
// What is checked, for each mask given as CSR lists (sorted columns, one
// emask index each):
//   - jaccard agrees with a set computation;
//   - build_pairs pairs exactly the rows its rule names (replayed here on
//     sets: rows in order, partner r + 1 or r + s / 128 of larger Jaccard
//     overlap, first on ties, if above 0);
//   - chunk_order keeps each chunk's items and sorts them by decreasing
//     weight, ties in order;
//   - build_pairs covers every row exactly once, pairs a row only with
//     r + 1 or r + s / 128, lists for each pair the ascending union of its
//     members' blocks with each member's own emask index (kAbsent where it
//     does not keep the block), and orders the pairs chunk-wise heaviest
//     first;
//   - transpose_csr lists, per column, the rows that keep it in ascending
//     order with the same emask indices.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "tra_sched.h"

namespace {

int g_checks = 0;

#define CHECK(cond, ...)                                              \
    do {                                                              \
        ++g_checks;                                                   \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n  ", __FILE__, __LINE__, #cond); \
            fprintf(stderr, __VA_ARGS__);                             \
            fprintf(stderr, "\n");                                    \
            exit(1);                                                  \
        }                                                             \
    } while (0)

struct Csr {
    int nrows = 0, ncols = 0;
    std::vector<int32_t> ptr, col, em;
};

Csr random_csr(std::mt19937_64 &rng, int nrows, int ncols, double density)
{
    Csr m;
    m.nrows = nrows;
    m.ncols = ncols;
    m.ptr.push_back(0);
    std::uniform_real_distribution<double> u(0.0, 1.0);
    int partial = 0;
    for (int r = 0; r < nrows; ++r) {
        for (int c = 0; c < ncols; ++c)
            if (u(rng) < density) {
                m.col.push_back(c);
                m.em.push_back(u(rng) < 0.3 ? partial++ : -1);
            }
        m.ptr.push_back((int32_t)m.col.size());
    }
    return m;
}

// Row r keeps the columns within `band` of r and of r -/+ k * per_frame
// (a radial-like pattern of frames of per_frame blocks).
Csr banded_csr(int nrows, int per_frame, int band, int frames_reach)
{
    Csr m;
    m.nrows = m.ncols = nrows;
    m.ptr.push_back(0);
    int partial = 0;
    for (int r = 0; r < nrows; ++r) {
        std::set<int> keep;
        for (int k = -frames_reach; k <= frames_reach; ++k)
            for (int d = -band; d <= band; ++d) {
                const int c = r + k * per_frame + d;
                if (c >= 0 && c < nrows)
                    keep.insert(c);
            }
        for (int c : keep) {
            m.col.push_back(c);
            m.em.push_back(((r + c) % 5 == 0) ? partial++ : -1);
        }
        m.ptr.push_back((int32_t)m.col.size());
    }
    return m;
}

void check_jaccard(std::mt19937_64 &rng)
{
    for (int t = 0; t < 200; ++t) {
        std::set<int32_t> a, b;
        const int na = (int)(rng() % 40), nb = (int)(rng() % 40);
        for (int i = 0; i < na; ++i)
            a.insert((int32_t)(rng() % 60));
        for (int i = 0; i < nb; ++i)
            b.insert((int32_t)(rng() % 60));
        std::vector<int32_t> va(a.begin(), a.end()), vb(b.begin(), b.end());
        std::vector<int32_t> inter, uni;
        std::set_intersection(va.begin(), va.end(), vb.begin(), vb.end(), std::back_inserter(inter));
        std::set_union(va.begin(), va.end(), vb.begin(), vb.end(), std::back_inserter(uni));
        const double want = uni.empty() ? 1.0 : (double)inter.size() / (double)uni.size();
        const double got = tra::jaccard(va.data(), (int)va.size(), vb.data(), (int)vb.size());
        CHECK(got == want, "jaccard %g, want %g", got, want);
    }
}

void check_chunk_order(std::mt19937_64 &rng)
{
    for (int t = 0; t < 50; ++t) {
        const int n = (int)(rng() % 300), chunk = 1 + (int)(rng() % 70);
        std::vector<int64_t> w(n);
        for (auto &x : w)
            x = (int64_t)(rng() % 6);
        const std::vector<int32_t> ord = tra::chunk_order(w, chunk);
        CHECK((int)ord.size() == n, "size %d", (int)ord.size());
        for (int i = 0; i < n; ++i) {
            CHECK(ord[i] >= 0 && ord[i] < n && ord[i] / chunk == i / chunk, "item %d at %d", ord[i], i);
            if (i % chunk != 0) {
                const int64_t wp = w[ord[i - 1]], wi = w[ord[i]];
                CHECK(wp > wi || (wp == wi && ord[i - 1] < ord[i]), "order at %d", i);
            }
        }
        std::vector<int32_t> sorted(ord);
        std::sort(sorted.begin(), sorted.end());
        for (int i = 0; i < n; ++i)
            CHECK(sorted[i] == i, "not a permutation at %d", i);
    }
}

void check_pairs(const Csr &m, int64_t s, const char *what)
{
    const tra::PairSchedule ps = tra::build_pairs(m.nrows, s, m.ptr, m.col, m.em);
    CHECK(ps.rows.size() % 2 == 0, "%s: odd member list", what);
    const int np = (int)ps.rows.size() / 2;
    CHECK((int)ps.ptr.size() == np + 1 && ps.ptr[0] == 0 && ps.ptr[np] == (int32_t)ps.col.size(),
          "%s: pair offsets", what);
    CHECK(ps.em.size() == 2 * ps.col.size(), "%s: emask list size", what);
    const int step = (s % tra::kBlock == 0 && s / tra::kBlock > 1) ? (int)(s / tra::kBlock) : 1;
    std::vector<int> seen(m.nrows, 0);
    for (int p = 0; p < np; ++p) {
        const int a = ps.rows[2 * p], b = ps.rows[2 * p + 1];
        CHECK(a >= 0 && a < m.nrows, "%s: pair %d first member %d", what, p, a);
        ++seen[a];
        if (b >= 0) {
            CHECK(b < m.nrows && (b == a + 1 || b == a + step), "%s: pair %d = (%d, %d)", what, p, a, b);
            ++seen[b];
        } else {
            CHECK(b == -1, "%s: pair %d second member %d", what, p, b);
        }
        // the merged list is the ascending union, with each member's index
        std::map<int32_t, int32_t> ea, eb;
        for (int32_t e = m.ptr[a]; e < m.ptr[a + 1]; ++e)
            ea[m.col[e]] = m.em[e];
        if (b >= 0)
            for (int32_t e = m.ptr[b]; e < m.ptr[b + 1]; ++e)
                eb[m.col[e]] = m.em[e];
        std::set<int32_t> uni;
        for (auto &kv : ea)
            uni.insert(kv.first);
        for (auto &kv : eb)
            uni.insert(kv.first);
        CHECK(ps.ptr[p + 1] - ps.ptr[p] == (int32_t)uni.size(), "%s: pair %d union size", what, p);
        int32_t at = ps.ptr[p];
        for (int32_t c : uni) {
            CHECK(ps.col[at] == c, "%s: pair %d entry %d is %d, want %d", what, p, at, ps.col[at], c);
            const auto ia = ea.find(c), ib = eb.find(c);
            CHECK(ps.em[2 * at] == (ia == ea.end() ? tra::kAbsent : ia->second), "%s: pair %d em a", what, p);
            CHECK(ps.em[2 * at + 1] == (ib == eb.end() ? tra::kAbsent : ib->second), "%s: pair %d em b", what, p);
            ++at;
        }
    }
    for (int r = 0; r < m.nrows; ++r)
        CHECK(seen[r] == 1, "%s: row %d in %d pairs", what, r, seen[r]);
    // the pairing rule, replayed with sets: rows in order; an unpaired row
    // takes, among the unpaired rows r + 1 and r + step, the one of larger
    // Jaccard overlap (the first on ties) if that overlap is above 0
    {
        std::vector<std::set<int32_t>> sets(m.nrows);
        for (int r = 0; r < m.nrows; ++r)
            for (int32_t e = m.ptr[r]; e < m.ptr[r + 1]; ++e)
                sets[r].insert(m.col[e]);
        auto jac = [&](int a, int b) {
            std::vector<int32_t> inter, uni;
            std::set_intersection(sets[a].begin(), sets[a].end(), sets[b].begin(), sets[b].end(),
                                  std::back_inserter(inter));
            std::set_union(sets[a].begin(), sets[a].end(), sets[b].begin(), sets[b].end(), std::back_inserter(uni));
            return uni.empty() ? 1.0 : (double)inter.size() / (double)uni.size();
        };
        std::vector<char> used(m.nrows, 0);
        std::vector<std::pair<int, int>> want;
        for (int r = 0; r < m.nrows; ++r) {
            if (used[r])
                continue;
            int best = -1;
            double bj = 0.0;
            std::vector<int> offs = {1};
            if (step > 1)
                offs.push_back(step);
            for (int off : offs) {
                const int r2 = r + off;
                if (r2 < m.nrows && !used[r2] && jac(r, r2) > bj) {
                    bj = jac(r, r2);
                    best = r2;
                }
            }
            used[r] = 1;
            if (best >= 0)
                used[best] = 1;
            want.push_back({r, best});
        }
        CHECK((int)want.size() == np, "%s: %d pairs, the rule gives %d", what, np, (int)want.size());
        for (int p = 0; p < np; ++p)
            CHECK(ps.rows[2 * p] == want[p].first && ps.rows[2 * p + 1] == want[p].second,
                  "%s: pair %d = (%d, %d), the rule gives (%d, %d)", what, p, ps.rows[2 * p], ps.rows[2 * p + 1],
                  want[p].first, want[p].second);
    }
    // chunk-wise heaviest first
    std::vector<int64_t> w(np);
    for (int p = 0; p < np; ++p)
        w[p] = ps.ptr[p + 1] - ps.ptr[p];
    CHECK(ps.order == tra::chunk_order(w, tra::kPairChunk), "%s: pair order", what);
}

void check_transpose(const Csr &m, const char *what)
{
    std::vector<int32_t> cp, ri, et;
    tra::transpose_csr(m.nrows, m.ncols, m.ptr, m.col, m.em, cp, ri, et);
    CHECK((int)cp.size() == m.ncols + 1 && cp[0] == 0 && cp[m.ncols] == m.ptr[m.nrows], "%s: column offsets",
          what);
    std::set<std::tuple<int32_t, int32_t, int32_t>> want, got;
    for (int r = 0; r < m.nrows; ++r)
        for (int32_t e = m.ptr[r]; e < m.ptr[r + 1]; ++e)
            want.insert({r, m.col[e], m.em[e]});
    for (int c = 0; c < m.ncols; ++c) {
        CHECK(cp[c] <= cp[c + 1], "%s: column %d offsets", what, c);
        for (int32_t e = cp[c]; e < cp[c + 1]; ++e) {
            if (e > cp[c])
                CHECK(ri[e - 1] < ri[e], "%s: column %d rows not ascending", what, c);
            got.insert({ri[e], c, et[e]});
        }
    }
    CHECK(got == want, "%s: transposed blocks differ", what);
}

}  // namespace

int main()
{
    std::mt19937_64 rng(20251203);
    check_jaccard(rng);
    check_chunk_order(rng);
    const int64_t frame_sizes[] = {128, 256, 384, 1536, 200, 64};
    for (int t = 0; t < 60; ++t) {
        const int nrows = (int)(rng() % 140);
        const int ncols = 1 + (int)(rng() % 140);
        const double density = (t % 4) * 0.3;
        const Csr m = random_csr(rng, nrows, ncols, density);
        const int64_t s = frame_sizes[t % 6];
        char what[96];
        snprintf(what, sizeof what, "random #%d (%d x %d, density %.1f, s %lld)", t, nrows, ncols, density,
                 (long long)s);
        check_pairs(m, s, what);
        check_transpose(m, what);
    }
    for (int per_frame : {1, 2, 3, 8, 12}) {
        for (int band : {0, 1, 3}) {
            const Csr m = banded_csr(per_frame * 17 + 5, per_frame, band, 2);
            char what[96];
            snprintf(what, sizeof what, "banded (frame %d blocks, band %d)", per_frame, band);
            check_pairs(m, (int64_t)per_frame * tra::kBlock, what);
            check_transpose(m, what);
        }
    }
    printf("sched_check: %d checks passed\n", g_checks);
    return 0;
}

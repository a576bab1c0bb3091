// Host-side construction of the work schedules of a compiled mask.  Plain
// C++ with no HIP dependency, so that it also builds and runs on its own
// (the sanitizer checks of the tests compile it with g++).
#pragma once

#include <stdint.h>

#include <vector>

namespace tra {

constexpr int kBlock = 128;  // mask block edge (Radial Attention section 6)
// Work distribution: query blocks are grouped in chunks of kChunk consecutive
// blocks; chunk g of the (batch * head)-major chunk list belongs to the queue
// of XCD g % kQueues.
constexpr int kChunk = 64;      // query blocks per chunk (one per workgroup slot)
constexpr int kPairChunk = 32;  // query-block pairs per chunk

// Emask index of a union-schedule entry for a query block that does not keep
// the entry's key block.
constexpr int32_t kAbsent = -2;

// |A n B| / |A u B| of two ascending lists (1 for two empty lists).
double jaccard(const int32_t *a, int na, const int32_t *b, int nb);

// Within each run of `chunk` consecutive items, the items by decreasing
// weight (ties keep their order).
std::vector<int32_t> chunk_order(const std::vector<int64_t> &weight, int chunk);

// Pair schedule of a block mask given as CSR lists (row r keeps blocks
// col[ptr[r]] .. in ascending order, each with an emask index, -1 = full):
// greedy pairing of rows, in order, with the unpaired partner among r + 1
// and r + s / 128 (same position in the next frame) of larger Jaccard
// overlap, if the two share any block (a tile step that serves one member
// of a pair costs what a step of an unpaired row costs, and a shared block
// serves both, so any overlap pays); then the merged block list of each
// pair with one emask index per member (kAbsent where the member does not
// keep the block), and the chunk-wise heaviest-first pair order.
struct PairSchedule {
    std::vector<int32_t> rows;   // [npairs][2] member rows (second -1: unpaired)
    std::vector<int32_t> ptr;    // [npairs + 1] offsets into col / em
    std::vector<int32_t> col;    // merged block list of every pair
    std::vector<int32_t> em;     // [ncol][2] emask index per member
    std::vector<int32_t> order;  // pairs, chunk-wise heaviest first
};
PairSchedule build_pairs(int nrows, int64_t s, const std::vector<int32_t> &ptr, const std::vector<int32_t> &col,
                         const std::vector<int32_t> &em);

// Column lists of a CSR block mask with nrows rows and ncols columns: column
// c keeps rows row_idx[col_ptr[c]] .. in ascending order, with the emask
// index em_t of each block.
void transpose_csr(int nrows, int ncols, const std::vector<int32_t> &ptr, const std::vector<int32_t> &col,
                   const std::vector<int32_t> &em, std::vector<int32_t> &col_ptr, std::vector<int32_t> &row_idx,
                   std::vector<int32_t> &em_t);

}  // namespace tra

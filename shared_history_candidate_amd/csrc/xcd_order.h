// Work-group order of the head-pair kernels (32-wide heads over one K = V
// memory: one work-group per plan item and pair of heads).
//
// Work-groups go to the eight XCDs of the chip (each with its own L2) in
// turn, work-group b to XCD b % 8.  The plan lists the items of one request
// (its slots and candidate blocks, which all read the request's memory rows)
// one after another, so chunks of kXcdChunk consecutive items go to one XCD
// with the same head pair: XCD x takes head pair x % pairs and every
// (8 / pairs)-th chunk, in plan order, and a line read by one item of the
// chunk is in that XCD's L2 for the others.  (The plain order puts
// consecutive items of one head pair on alternate XCDs, and each line is
// fetched twice.)  Head counts whose pairs do not divide 8 keep the plain
// order.
//
// The plan is sorted longest memory first, and each XCD deals its
// work-groups to its compute units in turn, so without more care the first
// compute unit of an XCD would get the longest item of every round and the
// last one the shortest.  Every other round of kXcdRound work-groups per XCD
// (one per compute unit) therefore runs in reverse order: compute unit j
// takes positions j, 2 kXcdRound - 1 - j, 2 kXcdRound + j, ..., whose memory
// lengths sum to about the same for every j.  The grid covers whole rounds,
// so the reversal stays inside it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

constexpr int kXcds = 8, kXcdChunk = 8;
constexpr int kXcdRound = 32;   // compute units per XCD (MI355X: 256 in 8 XCDs)
static_assert(kXcdRound % kXcdChunk == 0, "a round holds whole chunks");

__host__ __device__ inline bool xcd_chunked(int pairs) {
    return pairs <= kXcds && kXcds % pairs == 0;
}

// Item and head pair of work-group b.  Work-groups past the plan's items
// get an item index the caller rejects against the plan's item count.
__device__ inline void xcd_pair_item(int b, int pairs, int& item, int& pair) {
    if (xcd_chunked(pairs)) {
        const int x = b % kXcds;
        int k = b / kXcds;
        const int r = k / kXcdRound;
        if (r & 1) k = r * kXcdRound + (kXcdRound - 1) - (k - r * kXcdRound);
        pair = x % pairs;
        item = ((k / kXcdChunk) * (kXcds / pairs) + x / pairs) * kXcdChunk + k % kXcdChunk;
    } else {
        item = b / pairs;
        pair = b - item * pairs;
    }
}

// Work-groups that cover max_items plan items in that order.
inline int64_t xcd_pair_grid(int64_t max_items, int pairs) {
    if (!xcd_chunked(pairs)) return max_items * pairs;
    const int64_t chunks = (max_items + kXcdChunk - 1) / kXcdChunk;
    const int64_t per = kXcds / pairs;
    const int64_t per_xcd = (chunks + per - 1) / per * kXcdChunk;   // work-groups per XCD
    return (per_xcd + kXcdRound - 1) / kXcdRound * kXcdRound * kXcds;
}

}  // namespace xattn

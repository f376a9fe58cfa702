// Varlen request/candidate planner (device side), shared by the standalone
// plan kernel and by the projection launch, which runs it in one extra
// work-group.
//
// Ragged batches are packed with no padding: each request r contributes
// q * ceil(N_r / tile_m) work items {r, s, c0, nc} (candidates [c0, c0+nc) of
// request r, query slot s).  Sources: ReST reading note (paper-archivist)
// s.5.5 (padding removal for variable-length sequences) and s.3.5 (one memory
// per request shared by all its candidates); HELIX card (ai-papers-daily,
// "Sequence Modeling"): padding-free variable-length execution.
//
// Order: requests by memory length L_r descending, ties by r ascending; inside
// a request, candidate blocks ascending and per block slots 0..q-1.  A tile's
// cost is proportional to nc * L_r, so the hardware's in-order dispatch of
// work-groups becomes longest-processing-time-first list scheduling.  With
// rank = false the requests stay in index order (the short-memory kernel,
// whose work-groups take equal shares of near-equal tiles, needs no ranking;
// any order is a valid plan for every attention kernel).
#pragma once

#include "common.h"

namespace xattn {

struct PlanSmem {
    alignas(16) int a[kPlanMaxRequests + 1];   // lengths, then tile counts, then tile starts
    int order[kPlanMaxRequests];     // requests in rank order
    int part[16];                    // wave totals of the scan (<= 1024 threads)
    int red;
};

template <int NT>
__device__ int plan_block_or(int v, int* red) {
    __syncthreads();
    if (threadIdx.x == 0) *red = 0;
    __syncthreads();
    if (v) atomicOr(red, v);
    __syncthreads();
    return *red;
}

// In-place exclusive scan of n (<= kPlanMaxRequests) ints; returns the total.
// Each thread sums kPer consecutive entries; the per-thread sums are scanned
// inside each wave with shuffles, then across the NT / 64 wave totals.
template <int NT>
__device__ int plan_exclusive_scan(int* a, int n, int* part) {
    constexpr int kPer = kPlanMaxRequests / NT;
    constexpr int kWaves = NT / 64;
    static_assert(kWaves <= 16, "one wave total per scan slot");
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int sum = 0;
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        sum += (k < n) ? a[k] : 0;
    }
    int inc = sum;   // inclusive scan over the wave's lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(inc, off, 64);
        if (lane >= off) inc += v;
    }
    if (lane == 63) part[wv] = inc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int p = part[i];
        base += i < wv ? p : 0;
        total += p;
    }
    int run = base + inc - sum;
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        if (k < n) {
            const int c = a[k];
            a[k] = run;
            run += c;
        }
    }
    __syncthreads();
    return total;
}

// Compare-exchange of a bitonic sorting network (descending overall): the
// element at position i keeps the larger key when it is the lower one of its
// pair in a block that sorts descending, or the upper one in a block that
// sorts ascending.
__device__ __forceinline__ uint64_t plan_cx(uint64_t mine, uint64_t other, int i, int j, int k) {
    const bool keep_max = ((i & j) == 0) == ((i & k) == 0);
    return keep_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
}

// sm.order[p] = the request of rank p under (L_r descending, r ascending),
// for p < R.  Each request gets the key (L_r + 1) << 12 | (4095 - r), so the
// order is one unsigned comparison (keys are distinct; 0 pads), and the keys
// are sorted descending by a bitonic network over n = 2^m >= max(R, 64)
// positions: O(n log^2 n) work in log2(n) (log2(n) + 1) / 2 steps.
//   n <= NT: thread t holds position t in a register; partners closer than
//     64 are other lanes of its wave, farther ones come through LDS (only
//     those steps need a work-group barrier).
//   n > NT (large batches): the keys stay in LDS, one barrier per step.
template <int NT>
__device__ void plan_rank(const int* __restrict__ cu_kv, int R, PlanSmem& sm) {
    static_assert(kPlanMaxRequests <= 4096, "request index must fit 12 bits of the key");
    const int t = threadIdx.x;
    int n = 64;
    while (n < R) n <<= 1;
    uint64_t* ks = reinterpret_cast<uint64_t*>(sm.a);   // n keys over a[] and order[]
    auto key_of = [&](int i) -> uint64_t {
        return i < R ? ((uint64_t)(uint32_t)(cu_kv[i + 1] - cu_kv[i] + 1) << 12) |
                           (uint64_t)(4095 - i)
                     : 0;
    };
    if (n <= NT) {
        // waves past position n (n is a multiple of 64) only keep the barriers
        const bool holds = t < n;
        uint64_t key = key_of(t);
        for (int k = 2; k <= n; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                if (j >= 64) {
                    __syncthreads();   // the previous exchange's reads are done
                    if (holds) ks[t] = key;
                    __syncthreads();
                    if (holds) key = plan_cx(key, ks[t ^ j], t, j, k);
                } else if (holds) {
                    const uint32_t lo = __shfl_xor((uint32_t)key, j, 64);
                    const uint32_t hi = __shfl_xor((uint32_t)(key >> 32), j, 64);
                    key = plan_cx(key, ((uint64_t)hi << 32) | lo, t, j, k);
                }
            }
        }
        __syncthreads();   // keys held in registers; order[] is free
        if (t < R) sm.order[t] = 4095 - (int)(key & 4095);
        __syncthreads();
        return;
    }
    for (int i = t; i < n; i += NT) ks[i] = key_of(i);
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            __syncthreads();
            for (int p = t; p < n / 2; p += NT) {
                const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));   // lower position of pair p
                const uint64_t a = ks[i], b = ks[i + j];
                const uint64_t mx = a > b ? a : b, mn = a > b ? b : a;
                const bool desc = (i & k) == 0;
                ks[i] = desc ? mx : mn;
                ks[i + j] = desc ? mn : mx;
            }
        }
    }
    // order[] overlays the upper half of the keys: extract from the top, a
    // batch of NT positions at a time.  order[i] lands on key index
    // (4097 + i) / 2 or above, never on a position below the batch.
    for (int hi = (R + NT - 1) / NT * NT; hi > 0; hi -= NT) {
        const int i = hi - NT + t;
        __syncthreads();
        const uint64_t key = i < R ? ks[i] : 0;
        __syncthreads();
        if (i < R) sm.order[i] = 4095 - (int)(key & 4095);
    }
    __syncthreads();
}

// The whole plan in one work-group of NT threads: validate the offsets, rank
// the requests, scan the tile counts, write the tiles (and optionally cu_q,
// row_req and a copy of the tiles for the caller).
template <int NT>
__device__ void run_plan(const int* __restrict__ cu_kv, const int* __restrict__ cu_cand, int R,
                         int q, int tile_m, int total_cand, int total_kv, int* __restrict__ ws,
                         int64_t max_tiles, int* __restrict__ cu_q_out,
                         int* __restrict__ row_req_out, int* __restrict__ tiles_out,
                         int* __restrict__ n_tiles_out, PlanSmem& sm, bool rank = true) {
    const int t = threadIdx.x;

    // 1. Validate the offsets before anything is read through them.
    int err = 0;
    if (t == 0) {
        if (cu_kv[0] != 0 || cu_kv[R] != total_kv) err |= kErrCuKv;
        if (cu_cand[0] != 0 || cu_cand[R] != total_cand) err |= kErrCuCand;
    }
    for (int r = t; r < R; r += NT) {
        if (cu_kv[r + 1] < cu_kv[r]) err |= kErrCuKv;
        if (cu_cand[r + 1] < cu_cand[r]) err |= kErrCuCand;
    }
    err = plan_block_or<NT>(err, &sm.red);
    int4* tiles = reinterpret_cast<int4*>(reinterpret_cast<char*>(ws) + kPlanHeaderBytes);
    if (err) {
        if (t == 0) {
            ws[kPlanNTiles] = 0;
            ws[kPlanError] = err;
            ws[kPlanTileM] = tile_m;
            if (n_tiles_out) n_tiles_out[0] = 0;
        }
        return;
    }

    // 2. Rank requests by (L desc, r asc), or keep request order.
    if (rank) {
        plan_rank<NT>(cu_kv, R, sm);
    } else {
        for (int r = t; r < R; r += NT) sm.order[r] = r;
        __syncthreads();
    }

    // 3. Tile counts in ranked order (over the lengths, no longer needed),
    //    then their exclusive scan.
    for (int k = t; k < R; k += NT) {
        const int r = sm.order[k];
        const int n = cu_cand[r + 1] - cu_cand[r];
        sm.a[k] = q * ((n + tile_m - 1) / tile_m);
    }
    __syncthreads();
    const int total = plan_exclusive_scan<NT>(sm.a, R, sm.part);
    if (t == 0) sm.a[R] = total;
    __syncthreads();

    // 4. Write the tiles (total <= max_tiles because cu_cand[R] == total_cand).
    for (int i = t; i < total && i < max_tiles; i += NT) {
        int lo = 0, hi = R;  // largest k with a[k] <= i
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sm.a[mid] <= i) lo = mid; else hi = mid;
        }
        const int r = sm.order[lo];
        const int local = i - sm.a[lo];
        const int b = local / q, s = local - b * q;
        const int n = cu_cand[r + 1] - cu_cand[r];
        const int c0 = cu_cand[r] + b * tile_m;
        const int nc = min(tile_m, n - b * tile_m);
        const int kv0 = cu_kv[r];
        tiles[i] = make_int4(kv0, cu_kv[r + 1] - kv0, c0, nc | (s << 16));
        if (tiles_out) reinterpret_cast<int4*>(tiles_out)[i] = make_int4(r, s, c0, nc);
    }
    if (t == 0) {
        ws[kPlanNTiles] = total;
        ws[kPlanError] = 0;
        ws[kPlanTileM] = tile_m;
        if (n_tiles_out) n_tiles_out[0] = total;
    }

    // 5. Optional row maps (plan entry point only).
    if (cu_q_out)
        for (int r = t; r <= R; r += NT) cu_q_out[r] = q * cu_cand[r];
    if (row_req_out) {
        const int rows = q * total_cand;
        for (int row = t; row < rows; row += NT) {
            const int c = row / q;
            int lo = 0, hi = R;  // largest r with cu_cand[r] <= c (skips empty requests)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (cu_cand[mid] <= c) lo = mid; else hi = mid;
            }
            row_req_out[row] = lo;
        }
    }
}

}  // namespace xattn

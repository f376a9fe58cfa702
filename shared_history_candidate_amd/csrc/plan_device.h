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
// work-groups becomes longest-processing-time-first list scheduling.
#pragma once

#include "common.h"

namespace xattn {

struct PlanSmem {
    int a[kPlanMaxRequests + 1];     // lengths, then tile counts, then tile starts
    int order[kPlanMaxRequests];     // requests in rank order
    int part[1024];                  // per-thread partial sums of the scan
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
template <int NT>
__device__ int plan_exclusive_scan(int* a, int n, int* part) {
    constexpr int kPer = kPlanMaxRequests / NT;
    const int t = threadIdx.x;
    int sum = 0;
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        sum += (k < n) ? a[k] : 0;
    }
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {   // Hillis-Steele over the partials
        const int v = (t >= off) ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = part[t] - sum;
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        if (k < n) {
            const int c = a[k];
            a[k] = run;
            run += c;
        }
    }
    const int total = part[NT - 1];
    __syncthreads();
    return total;
}

// The whole plan in one work-group of NT threads: validate the offsets, rank
// the requests, scan the tile counts, write the tiles (and optionally cu_q,
// row_req and a copy of the tiles for the caller).
template <int NT>
__device__ void run_plan(const int* __restrict__ cu_kv, const int* __restrict__ cu_cand, int R,
                         int q, int tile_m, int total_cand, int total_kv, int* __restrict__ ws,
                         int64_t max_tiles, int* __restrict__ cu_q_out,
                         int* __restrict__ row_req_out, int* __restrict__ tiles_out,
                         int* __restrict__ n_tiles_out, PlanSmem& sm) {
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

    // 2. Rank requests by (L desc, r asc).
    for (int r = t; r < R; r += NT) sm.a[r] = cu_kv[r + 1] - cu_kv[r];
    __syncthreads();
    for (int r = t; r < R; r += NT) {
        const int L = sm.a[r];
        int rank = 0;
        for (int k = 0; k < R; ++k) {
            const int Lk = sm.a[k];
            rank += (Lk > L) || (Lk == L && k < r);
        }
        sm.order[rank] = r;
    }
    __syncthreads();

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

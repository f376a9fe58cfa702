// Varlen request/candidate planner.
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
//
// One work-group of 1024 threads does the whole plan: validation of the
// offset arrays, ranking requests by (L desc, r asc), an exclusive scan of the
// per-request tile counts, and a parallel write of the tiles.
#include "common.h"
#include "internal.h"

namespace xattn {

namespace {

constexpr int kThreads = 1024;

__device__ int block_or(int v, int* red) {
    __syncthreads();
    if (threadIdx.x == 0) red[0] = 0;
    __syncthreads();
    if (v) atomicOr(red, v);
    __syncthreads();
    return red[0];
}

// In-place exclusive scan of n (<= 4*kThreads) ints in LDS; returns the total.
__device__ int block_exclusive_scan(int* a, int n, int* part) {
    const int t = threadIdx.x;
    constexpr int kPer = kPlanMaxRequests / kThreads;  // 4
    int loc[kPer];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        loc[u] = (k < n) ? a[k] : 0;
        sum += loc[u];
    }
    part[t] = sum;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread sums.
    for (int off = 1; off < kThreads; off <<= 1) {
        const int v = (t >= off) ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = part[t] - sum;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int k = t * kPer + u;
        if (k < n) a[k] = run;
        run += loc[u];
    }
    const int total = part[kThreads - 1];
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(
    const int* __restrict__ cu_kv, const int* __restrict__ cu_cand, int R, int q,
    int tile_m, int total_cand, int total_kv, int* __restrict__ ws, int64_t max_tiles,
    int* __restrict__ cu_q_out, int* __restrict__ row_req_out, int* __restrict__ tiles_out,
    int* __restrict__ n_tiles_out) {
    __shared__ int s_len[kPlanMaxRequests];
    __shared__ int s_order[kPlanMaxRequests];
    __shared__ int s_start[kPlanMaxRequests + 1];
    __shared__ int s_part[kThreads];
    __shared__ int s_red[1];
    const int t = threadIdx.x;

    // 1. Validate the offsets before anything is read through them.
    int err = 0;
    if (t == 0) {
        if (cu_kv[0] != 0 || cu_kv[R] != total_kv) err |= kErrCuKv;
        if (cu_cand[0] != 0 || cu_cand[R] != total_cand) err |= kErrCuCand;
    }
    for (int r = t; r < R; r += kThreads) {
        if (cu_kv[r + 1] < cu_kv[r]) err |= kErrCuKv;
        if (cu_cand[r + 1] < cu_cand[r]) err |= kErrCuCand;
    }
    err = block_or(err, s_red);
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
    for (int r = t; r < R; r += kThreads) s_len[r] = cu_kv[r + 1] - cu_kv[r];
    __syncthreads();
    for (int r = t; r < R; r += kThreads) {
        const int L = s_len[r];
        int rank = 0;
        for (int k = 0; k < R; ++k) {
            const int Lk = s_len[k];
            rank += (Lk > L) || (Lk == L && k < r);
        }
        s_order[rank] = r;
    }
    __syncthreads();

    // 3. Tile counts in ranked order, exclusive scan.
    for (int k = t; k < R; k += kThreads) {
        const int r = s_order[k];
        const int n = cu_cand[r + 1] - cu_cand[r];
        s_start[k] = q * ((n + tile_m - 1) / tile_m);
    }
    __syncthreads();
    const int total = block_exclusive_scan(s_start, R, s_part);
    if (t == 0) s_start[R] = total;
    __syncthreads();

    // 4. Write the tiles (total <= max_tiles because cu_cand[R] == total_cand).
    for (int i = t; i < total && i < max_tiles; i += kThreads) {
        int lo = 0, hi = R;  // largest k with s_start[k] <= i
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_start[mid] <= i) lo = mid; else hi = mid;
        }
        const int r = s_order[lo];
        const int local = i - s_start[lo];
        const int b = local / q, s = local - b * q;
        const int n = cu_cand[r + 1] - cu_cand[r];
        const int c0 = cu_cand[r] + b * tile_m;
        const int nc = min(tile_m, n - b * tile_m);
        const int4 rec = make_int4(r, s, c0, nc);
        tiles[i] = rec;
        if (tiles_out) reinterpret_cast<int4*>(tiles_out)[i] = rec;
    }
    if (t == 0) {
        ws[kPlanNTiles] = total;
        ws[kPlanError] = 0;
        ws[kPlanTileM] = tile_m;
        if (n_tiles_out) n_tiles_out[0] = total;
    }

    // 5. Optional row maps (plan entry point only).
    if (cu_q_out)
        for (int r = t; r <= R; r += kThreads) cu_q_out[r] = q * cu_cand[r];
    if (row_req_out) {
        const int rows = q * total_cand;
        for (int row = t; row < rows; row += kThreads) {
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

}  // namespace

hipError_t launch_plan(const int* cu_kv, const int* cu_cand, int R, int q, int tile_m,
                       int total_cand, int total_kv, void* ws, int64_t max_tiles, int* cu_q,
                       int* row_req, int* tiles, int* n_tiles, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, stream, cu_kv, cu_cand, R, q,
                       tile_m, total_cand, total_kv, static_cast<int*>(ws), max_tiles, cu_q,
                       row_req, tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace xattn

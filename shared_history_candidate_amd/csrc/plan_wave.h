// Varlen plan of a small batch (R <= 64 requests) computed by a single wave,
// one lane per request, with no LDS and no barrier.  It yields exactly the
// work items of the work-group planner (plan_device.h): requests ranked by
// memory length L_r descending (ties by r ascending), q * ceil(N_r / tile_m)
// items per request, candidate blocks ascending and slots 0..q-1 per block.
// The fused attention kernel runs it in every wave to find its own item, so a
// forward pass over a small batch is a single launch.
//
// Sources: ReST reading note (paper-archivist) s.5.5 (padding removal for
// variable-length sequences) and s.3.5 (one memory per request shared by all
// its candidates); HELIX card (ai-papers-daily, "Sequence Modeling"):
// padding-free variable-length execution.
#pragma once

#include "common.h"

namespace xattn {

// Per-lane view of the plan: lane r < R describes request r.
struct WavePlan {
    int err;      // validation bitmask (kErrCuKv | kErrCuCand), wave-uniform
    int total;    // number of work items, wave-uniform
    int kv0, L;   // request's first memory row and memory length
    int c_lo, N;  // request's first candidate and candidate count
    int start;    // index of the request's first work item
    int cnt;      // number of work items of the request
};

__device__ inline WavePlan wave_plan(const int* __restrict__ cu_kv,
                                     const int* __restrict__ cu_cand, int R, int q, int tile_m,
                                     int total_cand, int total_kv) {
    WavePlan p{};
    const int r = threadIdx.x & 63;
    const bool act = r < R;
    int kv_hi = 0, c_hi = 0;
    if (act) {
        p.kv0 = cu_kv[r];
        kv_hi = cu_kv[r + 1];
        p.c_lo = cu_cand[r];
        c_hi = cu_cand[r + 1];
    }
    // The offsets are checked before anything is read through them.
    const bool bad_kv =
        act && (kv_hi < p.kv0 || (r == 0 && p.kv0 != 0) || (r == R - 1 && kv_hi != total_kv));
    const bool bad_c =
        act && (c_hi < p.c_lo || (r == 0 && p.c_lo != 0) || (r == R - 1 && c_hi != total_cand));
    p.err = (__ballot(bad_kv) != 0 ? kErrCuKv : 0) | (__ballot(bad_c) != 0 ? kErrCuCand : 0);
    if (p.err) return p;
    p.L = kv_hi - p.kv0;
    p.N = c_hi - p.c_lo;
    p.cnt = act ? q * ((p.N + tile_m - 1) / tile_m) : 0;
    // rank by (L desc, r asc)
    int rank = 0;
    for (int k = 0; k < R; ++k) {
        const int Lk = __builtin_amdgcn_readlane(p.L, k);
        rank += (Lk > p.L) || (Lk == p.L && k < r);
    }
    // first item = work of every request ranked before this one
    int start = 0, total = 0;
    for (int k = 0; k < R; ++k) {
        const int rk = __builtin_amdgcn_readlane(rank, k);
        const int ck = __builtin_amdgcn_readlane(p.cnt, k);
        start += rk < rank ? ck : 0;
        total += ck;
    }
    p.start = start;
    p.total = total;
    return p;
}

// Work item i (wave-uniform, < total) in the workspace layout of
// plan_layout.h: {kv0, L, c0, nc | s << 16}.
__device__ inline int4 wave_plan_item(const WavePlan& p, int i, int q, int tile_m) {
    const bool hit = p.cnt > 0 && p.start <= i && i < p.start + p.cnt;
    const unsigned long long m = __ballot(hit);
    const int r = __builtin_amdgcn_readfirstlane(__ffsll((long long)m) - 1);
    const int local = i - __builtin_amdgcn_readlane(p.start, r);
    const int b = local / q, s = local - b * q;
    const int N = __builtin_amdgcn_readlane(p.N, r);
    return make_int4(__builtin_amdgcn_readlane(p.kv0, r), __builtin_amdgcn_readlane(p.L, r),
                     __builtin_amdgcn_readlane(p.c_lo, r) + b * tile_m,
                     min(tile_m, N - b * tile_m) | (s << 16));
}

// Write the plan (header and every work item) into the workspace, one wave.
__device__ inline void wave_plan_publish(const WavePlan& p, int R, int q, int tile_m,
                                         int* __restrict__ ws, int64_t max_tiles) {
    const int lane = threadIdx.x & 63;
    int4* items = reinterpret_cast<int4*>(reinterpret_cast<char*>(ws) + kPlanHeaderBytes);
    if (!p.err) {
        for (int i0 = 0; i0 < p.total; i0 += 64) {
            const int i = i0 + lane;
            int r = 0;
            for (int k = 0; k < R; ++k) {
                const int sk = __builtin_amdgcn_readlane(p.start, k);
                const int ck = __builtin_amdgcn_readlane(p.cnt, k);
                if (ck > 0 && sk <= i && i < sk + ck) r = k;
            }
            const int local = i - __shfl(p.start, r, 64);
            const int b = local / q, s = local - b * q;
            const int N = __shfl(p.N, r, 64);
            const int4 item = make_int4(__shfl(p.kv0, r, 64), __shfl(p.L, r, 64),
                                        __shfl(p.c_lo, r, 64) + b * tile_m,
                                        min(tile_m, N - b * tile_m) | (s << 16));
            if (i < p.total && i < max_tiles) items[i] = item;
        }
    }
    if (lane == 0) {
        ws[kPlanNTiles] = p.err ? 0 : p.total;
        ws[kPlanError] = p.err;
        ws[kPlanTileM] = tile_m;
    }
}

}  // namespace xattn

// Standalone varlen planner launch (xattn_plan): one work-group of 1024
// threads runs the planner of plan_device.h and also writes the row maps.
#include "internal.h"
#include "plan_device.h"

namespace xattn {

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void plan_kernel(
    const int* __restrict__ cu_kv, const int* __restrict__ cu_cand, int R, int q, int tile_m,
    int total_cand, int total_kv, int* __restrict__ ws, int64_t max_tiles,
    int* __restrict__ cu_q_out, int* __restrict__ row_req_out, int* __restrict__ tiles_out,
    int* __restrict__ n_tiles_out, int rank) {
    __shared__ PlanSmem sm;
    run_plan<kThreads>(cu_kv, cu_cand, R, q, tile_m, total_cand, total_kv, ws, max_tiles, cu_q_out,
                       row_req_out, tiles_out, n_tiles_out, sm, rank != 0);
}

}  // namespace

hipError_t launch_plan(const int* cu_kv, const int* cu_cand, int R, int q, int tile_m,
                       int total_cand, int total_kv, void* ws, int64_t max_tiles, int* cu_q,
                       int* row_req, int* tiles, int* n_tiles, hipStream_t stream, bool rank) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, stream, cu_kv, cu_cand, R, q,
                       tile_m, total_cand, total_kv, static_cast<int*>(ws), max_tiles, cu_q,
                       row_req, tiles, n_tiles, rank ? 1 : 0);
    return hipGetLastError();
}

}  // namespace xattn

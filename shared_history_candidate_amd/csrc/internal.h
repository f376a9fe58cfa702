// Host-side launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

hipError_t launch_plan(const int* cu_kv, const int* cu_cand, int R, int q, int tile_m,
                       int total_cand, int total_kv, void* ws, int64_t max_tiles, int* cu_q,
                       int* row_req, int* tiles, int* n_tiles, hipStream_t stream);

// bf16 attention over projected queries Qp [total_cand][q][d].  A
// work-group has rb x ksplit waves: rb query blocks of 32 candidates (tile_m
// = 32 * rb) and ksplit memory splits merged on chip.  attn_bf16_variant_smem
// returns the LDS bytes of variant (rb, ksplit) for head width dh and the
// K/V mode, 0 if not built.
int attn_bf16_variant_smem(int dh, int rb, int ksplit, bool sep);
hipError_t launch_attn_bf16(const void* Qp, const void* K, const void* V, const void* ws, int64_t max_tiles, int q, int d, int heads, int rb,
                            int ksplit, void* O, hipStream_t stream);

// bf16 TSP projection Q = Z W_Q[slot] into Qp; when ws is not NULL the same
// launch also runs the planner into ws (one extra work-group).
hipError_t launch_project_plan_bf16(const void* Z, const void* Wq, int total_cand, int q, int d,
                                    void* Qp, const int* cu_kv, const int* cu_cand, int R,
                                    int tile_m, int total_kv, void* ws, int64_t max_tiles,
                                    hipStream_t stream);

// fp32 path (tile_m = 64): attention over projected queries, projection.
hipError_t launch_attn_f32(const float* Qp, const float* K, const float* V, const void* ws, int64_t max_tiles, int q, int d, int heads, float* O,
                           hipStream_t stream);

hipError_t launch_project_f32(const float* Z, const float* Wq, int total_cand, int q, int d,
                              float* Q, hipStream_t stream);

}  // namespace xattn

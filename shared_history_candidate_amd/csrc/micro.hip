// Micro-benchmarks that bound the fused kernel on this chip: matrix-core
// issue rate, v_exp_f32 rate, LDS read bandwidth (plain and transposed) and
// HBM copy bandwidth.  They report "achievable" figures beside the vendor
// peaks; none of them is on the computation path.
//
// Each kernel runs a fixed, in-bounds loop and writes one value per thread so
// that the compiler keeps the work.  The host entry points time `reps`
// launches with HIP events on the caller's stream and return milliseconds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace xattn {
namespace {

// 8 independent accumulator chains per wave keep the matrix pipe busy.
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a[t] = (bf16)(0.001f * (lane + t));
        b[t] = (bf16)(0.002f * (lane - t));
    }
    f32x16 c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = mfma32(a, b, c[k]);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[k][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 16 independent exp2 chains per lane.
__global__ __launch_bounds__(256) void exp_loop(int iters, float* out) {
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = -0.001f * (threadIdx.x + k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = __builtin_amdgcn_exp2f(x[k]) - 1.0f;
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Independent fma chains: the plain fp32 VALU rate.
__global__ __launch_bounds__(256) void fma_loop(int iters, float* out) {
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = 0.001f * (threadIdx.x + k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = fmaf(x[k], 0.999f, 0.0001f);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS reads: mode 0 = ds_read_b64, 1 = ds_read_b128, 2 = transposed b64.
// Addresses stay inside a 32 KB buffer; the pattern is conflict-free rows.
template <int MODE>
__global__ __launch_bounds__(256) void lds_loop(int iters, float* out) {
    __shared__ __attribute__((aligned(16))) bf16 buf[16384];
    for (int i = threadIdx.x; i < 16384; i += 256) buf[i] = (bf16)(0.001f * (i & 255));
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc = 0.f;
    int base = wave * 4096 + lane * 8;  // element offset: 16 B per lane, wave-private 8 KB
    for (int i = 0; i < iters; ++i) {
        const int off = (base + (i & 7) * 512) & 16383;
        if constexpr (MODE == 0) {
            bf16x4 v = *reinterpret_cast<const bf16x4*>(buf + off);
            bf16x4 w = *reinterpret_cast<const bf16x4*>(buf + ((off + 4) & 16383));
            acc += (float)v[0] + (float)w[1];
        } else if constexpr (MODE == 1) {
            bf16x8 v = *reinterpret_cast<const bf16x8*>(buf + off);
            acc += (float)v[0] + (float)v[5];
        } else {
            bf16x4 v = lds_read_tr16(buf + off);
            bf16x4 w = lds_read_tr16(buf + ((off + 4) & 16383));
            acc += (float)v[0] + (float)w[1];
        }
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Grid-stride copy, U 16-byte loads in flight per lane before their stores,
// with nontemporal hints (the data is touched once).  Swept on MI355X over
// 256..8192 work-groups of 256 threads, U = 1..8, with and without the
// hints (1 GiB each way): one work-group per CU with four nontemporal loads
// in flight was the fastest, 6.0 TB/s (hipMemcpy: 5.2 TB/s).
template <int U>
__global__ void copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], b + i + u * stride);
    }
    for (; i < n; i += stride) b[i] = a[i];
}

// Reads the first 64 bytes of every 128-byte line (four lanes per line, 16
// bytes each): the access of a 64-byte head slice of 128-byte memory rows.
// One value per thread is written so that the loads are kept.
__global__ void half_line_read_kernel(const uint4* __restrict__ a, int64_t lines, float* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < lines * 4; i += stride) {
        const uint4 v = a[(i >> 2) * 8 + (i & 3)];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)acc;
}

template <typename F>
float time_ms(F launch, int reps, hipStream_t s) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
    launch();  // warm-up
    hipEventRecord(e0, s);
    for (int i = 0; i < reps; ++i) launch();
    hipEventRecord(e1, s);
    hipEventSynchronize(e1);
    float ms = -1.f;
    hipEventElapsedTime(&ms, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    return hipGetLastError() == hipSuccess ? ms / reps : -1.f;
}

}  // namespace
}  // namespace xattn

extern "C" {

// kind: 0 mfma 32x32x16 bf16, 1 v_exp_f32, 2 fp32 fma, 3 LDS b64, 4 LDS b128,
// 5 LDS transposed b64.  `out` is device scratch of blocks*256 floats.
// Returns average milliseconds per launch (negative on error).
float xattn_micro_run(int kind, int blocks, int iters, int reps, float* out, void* stream) {
    using namespace xattn;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto go = [&](auto kern) {
        return time_ms([&] { hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, iters, out); },
                       reps, s);
    };
    switch (kind) {
        case 0: return go(mfma_loop);
        case 1: return go(exp_loop);
        case 2: return go(fma_loop);
        case 3: return go(lds_loop<0>);
        case 4: return go(lds_loop<1>);
        case 5: return go(lds_loop<2>);
        default: return -1.f;
    }
}

// Device-to-device copy of `bytes` (multiple of 16) from a to b.
float xattn_micro_copy(const void* a, void* b, int64_t bytes, int reps, void* stream) {
    using namespace xattn;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = bytes / 16;
    return time_ms([&] {
        hipLaunchKernelGGL(copy_kernel<4>, dim3(256), dim3(256), 0, s,
                           static_cast<const u32x4*>(a), static_cast<u32x4*>(b), n);
    }, reps, s);
}

// Reads the first 64 bytes of each 128-byte line of `bytes` (a multiple of
// 128) at a; `out` is device scratch of 256 * 8 * 256 floats.  Returns
// average milliseconds per launch (negative on error).
float xattn_micro_half_line_read(const void* a, int64_t bytes, int reps, float* out, void* stream) {
    using namespace xattn;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bytes % 128 != 0 || bytes <= 0) return -1.f;
    return time_ms([&] {
        hipLaunchKernelGGL(half_line_read_kernel, dim3(256 * 8), dim3(256), 0, s,
                           static_cast<const uint4*>(a), bytes / 128, out);
    }, reps, s);
}

}  // extern "C"

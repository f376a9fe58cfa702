// Shared device-side definitions for the xattn HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_layout.h"

namespace xattn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 32x32x16 bf16 matrix-core product, fp32 accumulate (gfx950).
// Operand layout (lane l, t = 0..7): A[l%32][8*(l/32)+t], B[8*(l/32)+t][l%32].
// Result layout (lane l, reg r):   C[(r/4)*8 + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS transposed read of four 16-bit values.  Within each group of 16 lanes,
// lane i receives element (i%4) of the 8-byte chunks addressed by lanes
// 4u + i/4, u = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ float xor32(float v) {
    return __shfl_xor(v, 32, 64);
}

}  // namespace xattn

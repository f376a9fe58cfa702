// Direct global-to-LDS loads (gfx950 buffer loads with the lds modifier).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xattn {

// One direct global-to-LDS load: every lane's 16 bytes at byte offset voff of
// the buffer land in LDS at lds_addr + 16 * lane (out-of-range offsets land
// as zeros).  Written out (M0 set in the same block) because the compiler,
// seeing an LDS-writing load, would make the next LDS read of any buffer wait
// for it; the kernels instead wait for these loads explicitly (s_waitcnt
// vmcnt) before the barrier that publishes the data, and before the buffer
// is reused for anything else.  The load writes no register.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace xattn

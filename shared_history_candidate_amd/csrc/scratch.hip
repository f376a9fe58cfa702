// Library-owned device scratch for xattn_forward_noalloc: a file-scope
// device array that takes the place of the caller's workspace (plan header
// and items, and the projected queries on the paths that stage them).
//
// On the host, `scratch` names a host-side stand-in of the device variable,
// not a device address.  Its device address is resolved with
// hipGetSymbolAddress once per device, with that device current, and only
// that address is ever handed to kernels.  Every GPU holds its own copy of
// the array, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "xattn.h"

namespace xattn {

namespace {

static_assert(XATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) char scratch[XATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t scratch_capacity() { return XATTN_NOALLOC_SCRATCH_BYTES; }

hipError_t scratch_on_device(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;   // the caller makes it current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[device] = p;
    }
    *out = g_ptr[device];
    return hipSuccess;
}

}  // namespace xattn

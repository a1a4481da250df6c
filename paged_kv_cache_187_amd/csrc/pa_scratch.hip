// Fixed device scratch for the decode entry point that allocates nothing.
//
// The workspace of the split decode (partial maxima, sums and V sums) lives in one
// file-scope device array of PA_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on
// holds its own copy at its own address for the life of the process.  Host code never
// passes the array's name to a kernel (on the host that name is only a stand-in for the
// symbol): the first call on a device, with that device current, resolves the device
// address with hipGetSymbolAddress and keeps it; kernels get that address as their
// workspace pointer.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pagedattn.h"
#include "pa_internal.h"

namespace pa {

namespace {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device id (null: not resolved yet)
std::mutex g_scratch_mutex;

}  // namespace

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace pa

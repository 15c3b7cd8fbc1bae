// Static device scratch for the forward entry point that allocates nothing
// (kda_fwd_noalloc): the two-pass forward's record workspace, in a file-scope
// device array instead of memory the caller or the library allocates.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from module load until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address is looked
// up once per device (with that device current) by hipGetSymbolAddress and kept
// here; only that address is ever passed to kernels.  Every call on a GPU shares
// its array, so calls that overlap on one GPU (two streams, two host threads)
// race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_kernel.h"

namespace kda {

namespace {

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda

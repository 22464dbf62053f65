// Device-resident scratch for the allocation-free mask entry point
// (nabla_build_mask_raster_noalloc): a file-scope device array that every GPU the library
// runs on holds from module load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol); it asks
// the runtime once per device for the array's address on that device and hands out that
// address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nabla_internal.h"

namespace nabla {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t device_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // with this device current: its own copy of the array, at its own address
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace nabla

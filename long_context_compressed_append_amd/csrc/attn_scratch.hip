// The scratch array of lcca_sparse_attn_fwd_noalloc: the split partial
// softmax states of the attention, for callers that cannot allocate device
// memory.  A file-scope device array: every GPU the library runs on holds its
// own copy, at its own address, from the module's load until the process
// ends.  In host code `scratch` names a host-side stand-in, so its device
// address is looked up once per device (with that device current) and kept;
// only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lcca.h"

static __device__ __align__(256) unsigned char scratch[LCCA_ATTN_SCRATCH_BYTES];

namespace lcca {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

size_t attn_scratch_bytes() { return LCCA_ATTN_SCRATCH_BYTES; }

hipError_t attn_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace lcca

// The library's file-scope device memory:
//   * `scratch`, the array of lcca_sparse_attn_fwd_noalloc: the split partial
//     softmax states of the attention, for callers that cannot allocate
//     device memory;
//   * `debug_err`, the device error word of debug builds (LCCA_DEBUG), where
//     kernels record index violations for lcca_debug_check().
// Every GPU the library runs on holds its own copy of each, at its own
// address, from the module's load until the process ends.  In host code the
// names stand for host-side stand-ins, so their device addresses are looked
// up once per device (with that device current) and kept; only those
// addresses are ever passed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lcca.h"
#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[LCCA_ATTN_SCRATCH_BYTES];
#ifdef LCCA_DEBUG
static __device__ uint32_t debug_err;
#endif

namespace lcca {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
#ifdef LCCA_DEBUG
void* g_debug_ptr[kMaxDevices];
#endif
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

hipError_t debug_word(uint32_t** word) {
    *word = nullptr;
#ifdef LCCA_DEBUG
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_debug_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_err));
        if (e != hipSuccess) return e;
        g_debug_ptr[dev] = p;
    }
    *word = static_cast<uint32_t*>(g_debug_ptr[dev]);
#endif
    return hipSuccess;
}

}  // namespace lcca

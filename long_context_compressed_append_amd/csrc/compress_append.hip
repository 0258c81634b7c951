// compress_append kernel: grid (new token, slice); the device code is in
// compress_dev.h.
// [Page "vLLM uveo DeepSeek V4 s 8,7x manjim KV cacheom", section "Kako
//  funkcionira optimizacija KV cachea?": weighted summation of tokens.]
#include "compress_dev.h"

namespace lcca {

namespace {

template <int TOK>
__global__ __launch_bounds__(cmp::kThreads) void compress_append_kernel(CompressArgs p) {
    cmp::compress_append_body<TOK>(p, blockIdx.x, blockIdx.y);
}

}  // namespace

hipError_t launch_compress_append(const CompressArgs& a, int total_new, hipStream_t stream) {
    if (total_new <= 0) return hipSuccess;
    const int SK = (a.D + cmp::kSliceDims - 1) / cmp::kSliceDims;
    const int SI = a.ik_data != nullptr ? (a.dI + cmp::kSliceDims - 1) / cmp::kSliceDims : 0;
    dim3 grid(total_new, SK + SI + 1);
    if (a.tok_dtype == DT_F32)
        hipLaunchKernelGGL(compress_append_kernel<DT_F32>, grid, dim3(cmp::kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(compress_append_kernel<DT_BF16>, grid, dim3(cmp::kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lcca

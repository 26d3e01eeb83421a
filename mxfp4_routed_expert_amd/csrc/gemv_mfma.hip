// Decode down product and weighted combine on the matrix cores, MXFP4 weights (the body is
// in dm_body.h).
#include "dm_body.h"

namespace moe {

__global__ __launch_bounds__(kDmThreads) void down_combine_mfma_kernel(const DownCombineParams p) {
    dm_body<false>(p, blockIdx.x, blockIdx.y, nullptr, false);
}

void down_combine_mfma_launch(const DownCombineParams &p, dim3 grid, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL(down_combine_mfma_kernel, grid, dim3(kDmThreads), lds, stream, p);
}

}  // namespace moe

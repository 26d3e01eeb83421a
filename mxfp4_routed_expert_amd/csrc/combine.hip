// Atomic-free weighted combine of the routed expert rows and the shared expert.
//
// The layer's output is the routing-weighted sum of the selected experts' outputs plus
// the shared expert (rabbit README, design section; the "gated shared expert" of the
// architecture table).  Each output element is owned by one thread, which gathers its k
// rows through pair_to_row in the fixed order j = 0..k-1 and then adds the shared row:
// no atomics, so the result is bitwise reproducible.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(int T, int k, int d, int R, const float *__restrict__ y_rows,
                                                      const int32_t *__restrict__ p2r,
                                                      const float *__restrict__ topk_w,
                                                      const float *__restrict__ y_shared,
                                                      const float *__restrict__ sgate, float *__restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (c >= d) return;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool vec = (d & 3) == 0;
    for (int j = 0; j < k; ++j) {
        const int r = p2r[(size_t)t * k + j];
        const float w = topk_w[(size_t)t * k + j];
        if (r < 0 || r >= R) continue;
        const float *src = y_rows + (size_t)r * d + c;
        if (vec) {
            const f32x4 v = *(const f32x4 *)src;
            acc[0] = fmaf(w, v[0], acc[0]); acc[1] = fmaf(w, v[1], acc[1]);
            acc[2] = fmaf(w, v[2], acc[2]); acc[3] = fmaf(w, v[3], acc[3]);
        } else {
            for (int q = 0; q < 4 && c + q < d; ++q) acc[q] = fmaf(w, src[q], acc[q]);
        }
    }
    if (y_shared) {
        const float g = sgate ? sgate[t] : 1.0f;
        const float *src = y_shared + (size_t)t * d + c;
        for (int q = 0; q < 4 && c + q < d; ++q) acc[q] = fmaf(g, src[q], acc[q]);
    }
    float *dst = out + (size_t)t * d + c;
    if (vec) {
        *(f32x4 *)dst = acc;
    } else {
        for (int q = 0; q < 4 && c + q < d; ++q) dst[q] = acc[q];
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(int32_t T, int32_t k, int32_t d, const float *y_rows, const int32_t *pair_to_row,
                                  const float *topk_w, const float *y_shared, const float *shared_gate, float *out,
                                  moe_stream stream) {
    clear_error();
    MOE_REQUIRE(T >= 0 && d > 0 && k >= 0 && k <= MOE_MAX_TOPK, "moe_combine: need T >= 0, d > 0, 0 <= k <= %d",
                MOE_MAX_TOPK);
    MOE_REQUIRE((int64_t)T * d < INT32_MAX && (int64_t)T * k * d < INT32_MAX, "moe_combine: sizes overflow int32");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(out != nullptr, "moe_combine: NULL out");
    if (k > 0) MOE_REQUIRE(y_rows && pair_to_row && topk_w, "moe_combine: NULL y_rows, pair_to_row or topk_w");
    MOE_REQUIRE(!(shared_gate && !y_shared), "moe_combine: shared_gate given without y_shared");
    dim3 grid(((d + 3) / 4 + 255) / 256, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, (hipStream_t)stream, T, k, d, T * k, y_rows,
                       pair_to_row, topk_w, y_shared, shared_gate, out);
    return launch_check("moe_combine");
}

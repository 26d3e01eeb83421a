// Prefill grouped GEMM on the gfx950 block-scaled FP4 matrix instructions (placeholder:
// the GEMV path serves every shape until the MFMA kernels land).
#include "gemv.h"

namespace moe {

bool mfma_path_wanted(const moe_expert_weights *, int, int, int, bool) { return false; }

moe_status mfma_gateup_launch(const moe_expert_weights *, int, int, const uint8_t *, const uint8_t *,
                              const int32_t *, const int32_t *, int, float *, uint8_t *, uint8_t *, hipStream_t) {
    set_error("block-scaled FP4 grouped GEMM not available");
    return MOE_ERR_UNSUPPORTED;
}

moe_status mfma_down_launch(const moe_expert_weights *, const uint8_t *, const uint8_t *, const int32_t *, int,
                            float *, hipStream_t) {
    set_error("block-scaled FP4 grouped GEMM not available");
    return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe

// Declarations shared by the GEMV kernels (gemv.hip) and their callers.
#pragma once

#include "common.h"

namespace moe {

enum WFmt { kFmtMXFP4 = 0, kFmtFP8 = 1, kFmtBF16 = 2 };
enum ActKind { kActBF16 = 0, kActF32 = 1, kActMX = 2 };

struct GemvParams {
    const uint8_t *w[2];       // codes of the matrix (gate, up for the pair)
    const void *s[2];          // scales (MXFP4: u8 [E][N][K/32]; FP8: f32 [E][N/128][K/128])
    int N, K, E;               // rows per matrix, reduction length, experts in the stack
    const void *act;           // activation rows [n_act_rows][K] (bf16, f32, or MX codes [..][K/2])
    const uint8_t *act_s;      // MX activation scales [n_act_rows][K/32] (MX activations only)
    int gather;                // 1: activation row = sorted_pairs[r] / k; 0: activation row = r
    int n_act_rows;
    const int32_t *offsets;    // [E+1] or NULL: identity (expert 0, rows 0..T-1)
    const int32_t *sorted_pairs;
    int k;
    int T;                     // rows of the identity form
    int R;                     // rows of the output
    float *out;                // [R][N]
    const float *residual;     // [R][N] or NULL
    int G;                     // lanes per matrix row (power of two, <= 32 for the pair)
    int nl;                    // 16-byte units per lane per row
    int rows_per_wg;           // matrix rows per workgroup
    int chunk;                 // tokens staged in LDS at once (<= MAXM)
    int lds_ld;                // LDS row stride in elements (matrix-core GEMV)
};

// Enqueue one GEMV launch.  `slots` is the number of expert slots in the grid (experts
// that may own rows; 1 for the identity form); `max_rows_per_expert` bounds M_e and
// picks the register tile of tokens.
moe_status gemv_launch(int fmt, int act, bool pair, GemvParams p, int slots, int max_rows_per_expert,
                       hipStream_t stream, const char *what);

// Matrix-core decode GEMV (MXFP4 weights, N % 16 == 0); see gemv_mfma.hip.
bool gemv_mfma_supported(int fmt, const GemvParams &p);
moe_status gemv_mfma_launch(int act, bool pair, GemvParams p, int slots, hipStream_t stream, const char *what);

moe_status mx_quantize_launch(int rows, int cols, const void *x, bool f32, uint8_t *codes, uint8_t *scales,
                              hipStream_t stream);

}  // namespace moe

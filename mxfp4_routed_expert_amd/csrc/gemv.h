// Declarations shared by the GEMV kernels (gemv.hip) and their callers.
#pragma once

#include "common.h"

namespace moe {

enum WFmt { kFmtMXFP4 = 0, kFmtFP8 = 1, kFmtBF16 = 2 };
enum ActKind { kActBF16 = 0, kActF32 = 1, kActMX = 2 };

// Routing done by the decode gate/up kernel itself (moe_route_gateup_shared): the router's
// logits in, the routing results out (written by workgroup 0; every workgroup selects the
// same experts from the same logits).
struct RouteArgs {
    const float *logits = nullptr;  // [T][rows]: E expert logits, then the shared-gate logit
    int rows = 0, score = 0, renorm = 0, has_sg = 0, n_group = 1, topk_group = 1;
    float scaling = 1.0f;
    const float *lbias = nullptr, *sbias = nullptr;
    int32_t *ids = nullptr;
    float *tw = nullptr, *sg = nullptr;
    int32_t *offsets = nullptr, *sorted = nullptr, *p2r = nullptr;
};

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
    // Optional extra grid slot (grid y == shared_slot) that runs a second weight set over
    // the identity rows 0..T-1 -- the shared expert fused into the routed launch.
    int shared_slot = -1;      // -1: none
    const uint8_t *sw[2] = {nullptr, nullptr};
    const void *ss[2] = {nullptr, nullptr};
    int sN = 0;
    float *sout = nullptr;     // [T][sN]
    RouteArgs route;           // the routing-in-the-prologue form only
};

// Down product and weighted combine of decode-sized batches in one launch (gemv.hip):
//   out[t][n] = sum_j tw[t][j] * (W_down[ids[t][j]][n] . h[p2r[t*k+j]])
//               + g[t] * (W_shared_down[n] . hs[t])        (g = sg[t], or 1 when sg == NULL)
struct DownCombineParams {
    const uint8_t *w;          // routed down codes [E][N][I/2] (MXFP4) or [E][N][I] (FP8)
    const void *s;             // routed down scales
    const uint8_t *sw;         // shared down codes [N][I/..] or NULL
    const void *ss;
    int E, N, I;               // experts, output rows (d_model), reduction length (d_ff)
    const float *h;            // routed h rows [R][I] (sorted-pair order)
    const float *hs;           // shared h [T][I] or NULL
    const int32_t *ids;        // [T][k]
    const float *tw;           // [T][k]
    const int32_t *p2r;        // [T*k]
    const float *sg;           // [T] or NULL
    int T, k, R;
    float *out;                // [T][N]
    int G, nl, rows_per_wg;
    int h_lds_bytes;           // LDS bytes of the staged h rows (the table follows)
};
moe_status down_combine_launch(int fmt, DownCombineParams p, hipStream_t stream);
size_t down_combine_lds(int k, bool shared, int I);
// Down-combine launch shape: 512 threads; at most kDcMaxRows output rows per workgroup.
// A slot's h occupies 4 * dc_plane_ld(I) bytes of LDS (a multiple of 2 KiB): the float32 row,
// or bf16 hi + lo planes of dc_plane_ld(I) values (whole steps of 512 of the matrix-core form).
constexpr int kDcThreads = 512;
constexpr int kDcMaxRows = 128;
// The matrix-core (MXFP4) form keeps two partial sums per (slot, row): at most 64 rows.
constexpr int kDmMaxRows = kDcMaxRows / 2;
__host__ __device__ constexpr int dc_plane_ld(int I) { return (I + 511) / 512 * 512; }
void down_combine_mfma_launch(const DownCombineParams &p, dim3 grid, size_t lds, hipStream_t stream);

// Enqueue one GEMV launch.  `slots` is the number of expert slots in the grid (experts
// that may own rows; 1 for the identity form); `max_rows_per_expert` bounds M_e and
// picks the register tile of tokens.
moe_status gemv_launch(int fmt, int act, bool pair, GemvParams p, int slots, int max_rows_per_expert,
                       hipStream_t stream, const char *what);
// The decode gate/up (+ shared) launch that also routes (top-k and permutation of p.route's
// logits in every workgroup), bf16 activations: false when the shapes do not allow it
// (T > 4, T*k > 64, E > 512, or activation rows too wide), else the launch status in *st.
bool gemv_route_launch(int fmt, int act, GemvParams p, int slots, hipStream_t stream, moe_status *st);


// The single-launch decode step (decode_step_kernel, gemv.hip): router logits, top-k with
// the routed and shared gate/up, down with the weighted combine, one persistent launch of
// one workgroup per compute unit whose phases hand over through the caller's sync buffer.
struct StepParams {
    GemvParams gu;             // the routing-in-the-prologue gate/up launch's parameters
    DownCombineParams dc;      // the down-combine's
    const uint16_t *x;         // bf16 [T][H]
    const uint16_t *wr;        // router rows bf16 [E][H]
    const uint16_t *wsg;       // shared-gate row bf16 [H] or NULL
    int T, H, E, rows;         // rows = E + (wsg != NULL): logit rows per token
    float *logits;             // [T][rows]
    uint32_t *sync;            // the caller's sync buffer
    int nx;                    // down-combine row ranges per token
};
// Enqueues the step as one launch: false when the shapes do not allow it (the gate/up or
// down-combine forms do not take them, or one workgroup per CU does not fit), else the
// launch status in *st.
bool decode_step_launch(StepParams sp, hipStream_t stream, moe_status *st);

// route.hip: the routing arguments' checks of moe_route, and the selection (top-k, weights,
// permutation) of moe_route_permute from logits
// already computed (the first T*(E + has_sg) floats of `ws`).
moe_status check_route_desc(const moe_route_desc *d);
moe_status route_select_step(const moe_route_desc *d, const void *ws, const float *logit_bias,
                             const float *select_bias, bool has_sg, int32_t *topk_ids, float *topk_w,
                             float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_to_row,
                             hipStream_t s);

// The router logits of T < 32 tokens with no workspace (route.hip).
moe_status router_logits_small(const moe_route_desc *d, const void *x, const void *w_router, const void *w_shared_gate,
                               float *logits, hipStream_t s);

moe_status mx_quantize_launch(int rows, int cols, const void *x, bool f32, uint8_t *codes, uint8_t *scales,
                              hipStream_t stream);

}  // namespace moe

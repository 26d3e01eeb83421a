/*
 * moe.h -- C ABI of the routed Mixture-of-Experts FFN layer over block-quantised
 * expert weights, for AMD Instinct MI355X (gfx950).
 *
 * The layer (rabbit README, design section and architecture table; Kimi K3 article,
 * architecture section): for each token a router scores every expert (softmax, or
 * noaux_tc sigmoid with a selection-only bias), keeps the top k and renormalises their
 * weights; tokens are grouped by expert; each selected expert, stored as OCP MXFP4
 * (32-element E2M1 blocks sharing one E8M0 scale) or FP8 E4M3 with 128x128 block
 * scales, computes a SwiGLU FFN; a (gated) shared expert runs on every token; the
 * outputs are summed with the routing weights.  LatentMoE layers run the routed
 * experts at a narrower width between two bf16 projections.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, owned by the
 *     caller.  Descriptor structs are host memory, read during the call only.
 *   - Inputs are read-only and must not alias outputs.  Outputs are fully overwritten.
 *   - The library allocates no device memory.  Calls that need scratch space take a
 *     caller-owned workspace (query its size with the matching *_workspace call); its
 *     contents are undefined after the call.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without synchronising.  Calls are thread-safe.
 *   - Arguments are validated on the host before anything is enqueued; on failure the
 *     call returns a non-zero status, enqueues nothing and moe_last_error() describes
 *     the problem.  A failed launch returns MOE_ERR_HIP.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - T == 0 (no tokens) is valid: the call returns MOE_OK and enqueues nothing.
 *   - Device-side values that index memory (expert ids, offsets, pair indices) are
 *     range-checked in the kernels; out-of-range entries are skipped, never followed.
 */
#ifndef MXFP4_ROUTED_EXPERT_MOE_H
#define MXFP4_ROUTED_EXPERT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size or enum value        */
    MOE_ERR_UNSUPPORTED = 2, /* valid request this library does not implement        */
    MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace size   */
    MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed            */
} moe_status;

enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_W_MXFP4 = 0, MOE_W_FP8_E4M3_B128 = 1 };
/* MOE_ACT_FLOAT: activations are used as given (bf16 x, float32 h): weight-only quantisation.
 * MOE_ACT_MXFP4: x and h are OCP-MX-quantised to MXFP4 per 32-block and the products run on
 *                the block-scaled FP4 matrix cores (MXFP4 weights only). */
enum { MOE_ACT_FLOAT = 0, MOE_ACT_MXFP4 = 1 };
enum { MOE_DT_BF16 = 0, MOE_DT_F32 = 1 };

typedef void *moe_stream; /* hipStream_t */

/* Maximum sizes accepted: k <= 16, E <= 2048, every int32 product of sizes < 2^31. */
#define MOE_MAX_TOPK 16
#define MOE_MAX_EXPERTS 2048

typedef struct {
    int32_t T;              /* tokens                                             */
    int32_t H;              /* hidden width, multiple of 32                       */
    int32_t E;              /* routed experts, 1 <= E <= MOE_MAX_EXPERTS          */
    int32_t k;              /* experts per token, 1 <= k <= min(E, 16)            */
    int32_t score;          /* MOE_SCORE_*                                        */
    int32_t renormalize;    /* 1: divide the selected weights by their sum        */
    float routed_scaling;   /* multiplies the final routing weights               */
    int32_t n_group;        /* expert groups for group-limited selection (0 or 1: none) */
    int32_t topk_group;     /* groups kept per token when n_group > 1              */
} moe_route_desc;

/*
 * moe_route -- router logits, scoring, top-k and renormalisation.
 * ("softmax top-10 of 512 + gated shared expert" and "noaux_tc sigmoid": rabbit README,
 * architecture table, "MoE routing" row.)
 *   l[t][e]  = float32 rounding of the exact dot product x[t] . w_router[e]
 *              (+ logit_bias[e], added in float64 after rounding)
 *   softmax: select the k largest l (descending, ties to the lower expert index);
 *            w = softmax probability of each selected expert, divided by the sum over
 *            the selected ones when renormalize != 0.
 *   sigmoid: s = sigmoid(l); select the k largest s + select_bias (bias used for
 *            selection only); w = s, divided by the selected sum when renormalize != 0.
 *   w *= routed_scaling.  Post-logit arithmetic runs in float64.
 *   Group-limited selection ("grouped routing", Kimi Linear, and noaux_tc: rabbit README,
 *   architecture table), when n_group > 1: experts e are in group e / (E / n_group); a
 *   group's score is the sum of its two largest selection keys (sigmoid) or its largest
 *   key (softmax), NaN keys counting as -inf; the topk_group best groups are kept (ties to
 *   the lower group) and the k experts are selected among theirs only.  Needs
 *   E % n_group == 0, n_group <= 64, E / n_group >= 2 for sigmoid, 1 <= topk_group <=
 *   n_group and topk_group * (E / n_group) >= k.  The weights are computed as above.
 *   shared_gate[t] = sigmoid(float32(x[t] . w_shared_gate)) when w_shared_gate != NULL.
 * x: bf16 [T][H].  w_router: bf16 [E][H].  logit_bias, select_bias: float32 [E] or NULL
 * (select_bias only with MOE_SCORE_SIGMOID).  w_shared_gate: bf16 [H] or NULL.
 * topk_ids: int32 [T][k] out.  topk_w: float32 [T][k] out.  shared_gate: float32 [T] out,
 * required iff w_shared_gate != NULL.
 * ws: moe_route_workspace(desc) bytes.
 */
moe_status moe_route(const moe_route_desc *desc, const void *x, const void *w_router,
                     const float *logit_bias, const float *select_bias,
                     const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                     float *shared_gate, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_route_workspace(const moe_route_desc *desc);

/*
 * moe_permute -- group the P = T*k (token, slot) pairs by expert with a stable counting
 * sort.  Pair p = t*k + j refers to topk_ids[t][j].
 *   expert_offsets[e] = number of pairs routed to experts < e   (int32 [E+1])
 *   sorted_pairs[r]   = the pairs, grouped by expert, ascending p within an expert (int32 [P])
 *   pair_to_row[p]    = r such that sorted_pairs[r] == p                              (int32 [P])
 * Deterministic: positions come from a stable rank, not from atomics.
 * Ids outside [0, E) are dropped; their pair_to_row entry is -1 and the unused tail
 * of sorted_pairs is -1.  With T == 0 the call still writes expert_offsets (all zero).
 * (Tokens grouped per expert: rabbit README features list, per-expert early drain;
 * one launch for a step's routed experts: Rulith Inference README, engine section.)
 */
moe_status moe_permute(int32_t T, int32_t k, int32_t E, const int32_t *topk_ids,
                       int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_to_row,
                       void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_permute_workspace(int32_t T, int32_t k, int32_t E);

/*
 * moe_route_permute -- moe_route followed by moe_permute of its topk_ids, in one call.
 * Arguments and results are exactly those of the two calls (same layouts, same errors,
 * same workspace: moe_route_workspace(desc) bytes).  With T <= 4 and T*k <= 64 (decode)
 * the permutation is written by the top-k kernel itself, one launch fewer.
 * (Routing and per-expert grouping as in moe_route and moe_permute above.)
 */
moe_status moe_route_permute(const moe_route_desc *desc, const void *x, const void *w_router,
                             const float *logit_bias, const float *select_bias,
                             const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                             float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                             int32_t *pair_to_row, void *ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_route_permute_noalloc -- moe_route_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are those of
 * moe_route_permute; the routing scratch (moe_route_workspace(desc) bytes) lives instead in
 * a static device array of 8 MiB inside the library, one per GPU, held until the process
 * ends.  A request needing more scratch than that returns MOE_ERR_UNSUPPORTED before
 * anything is enqueued.  The call allocates nothing.  Every call on a GPU uses that GPU's
 * one array: calls that overlap in time on the same GPU (different streams or threads)
 * race and must be ordered by the caller.
 */
moe_status moe_route_permute_noalloc(const moe_route_desc *desc, const void *x, const void *w_router,
                                     const float *logit_bias, const float *select_bias,
                                     const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                     float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                     int32_t *pair_to_row, moe_stream stream);

/*
 * Expert weights for E experts (or one shared expert), stacked along the expert axis.
 *   MOE_W_MXFP4:          gate, up: codes uint8 [E][d_ff][d_model/2], scales uint8 E8M0
 *                         [E][d_ff][d_model/32]; down: codes [E][d_model][d_ff/2], scales
 *                         [E][d_model][d_ff/32].  Element k of a row is the LOW nibble of
 *                         byte k/2 when k is even, the high nibble when odd; E2M1 codes;
 *                         scale byte b means 2^(b-127), b = 255 is NaN.  d_model and d_ff
 *                         are multiples of 32.
 *   MOE_W_FP8_E4M3_B128:  gate, up: codes uint8 E4M3 (OCP "FN") [E][d_ff][d_model], scales
 *                         float32 [E][d_ff/128][d_model/128]; down: codes [E][d_model][d_ff],
 *                         scales [E][d_model/128][d_ff/128].  d_model and d_ff are
 *                         multiples of 128.
 * ("native quantization read: OCP MXFP4 ... FP8 (E4M3, block-scale)": rabbit README,
 * architecture table.)
 */
typedef struct {
    int32_t format;       /* MOE_W_*                                  */
    int32_t num_experts;  /* E                                        */
    int32_t d_model;      /* input width of gate/up, output of down   */
    int32_t d_ff;         /* intermediate width                       */
    const uint8_t *gate, *up, *down;
    const void *gate_s, *up_s, *down_s;
} moe_expert_weights;

/*
 * moe_expert_ffn -- every expert's SwiGLU FFN on the rows routed to it.
 *   h = silu(gate . a) * (up . a),  silu(g) = g / (1 + exp(-g)),  y = down . h,
 *   float32 accumulation.  ("SituAndMul" activation of the Kimi K3 experts, rabbit README
 *   source tree, read as SiLU-and-multiply.)
 * Routed form (expert_offsets != NULL): rows r in [expert_offsets[e], expert_offsets[e+1])
 *   belong to expert e and read token sorted_pairs[r] / k;  y_rows is [T*k][d_model].
 * Identity form (expert_offsets == NULL, num_experts must be 1): row t reads token t;
 *   y_rows is [T][d_model].  This is the shared expert.
 * x: [T][d_model], x_dtype MOE_DT_BF16 or MOE_DT_F32.
 * act == MOE_ACT_FLOAT: weights are decoded exactly (an E2M1 code times its E8M0 scale is
 *   a bf16 value); x and h are used as given.  With MXFP4 weights and T >= 64 the products
 *   run on the bf16 matrix cores, a float32 operand (h, or float32 x) as the two bf16 terms
 *   hi = RN(v), lo = RN(v - hi), together within 2^-17 |v|; otherwise, and for FP8 weights,
 *   on the vector ALU in float32.
 * act == MOE_ACT_MXFP4: x and h are MX-quantised (OCP MX v1.0: scale 2^(floor(log2 amax)-2),
 *   round to nearest even, saturate at 6) and the products use the block-scaled FP4
 *   matrix instructions; MXFP4 weights only (else MOE_ERR_UNSUPPORTED).
 * ws: moe_expert_ffn_workspace(w, act, T, k) bytes (k ignored in the identity form).
 */
moe_status moe_expert_ffn(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k,
                          const void *x, int32_t x_dtype, const int32_t *expert_offsets,
                          const int32_t *sorted_pairs, float *y_rows, void *ws, size_t ws_bytes,
                          moe_stream stream);
size_t moe_expert_ffn_workspace(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k);

/*
 * The two stages of moe_expert_ffn, exposed separately (R = T*k rows routed, T identity).
 * moe_expert_gateup writes h = silu(gate . a) * (up . a):
 *   MOE_ACT_FLOAT: h float32 [R][d_ff] required; h_codes / h_scales ignored.
 *   MOE_ACT_MXFP4: h_codes uint8 [R][d_ff/2] and h_scales uint8 [R][d_ff/32] required (the
 *                  MX-quantised h); h (float32, before quantisation) optional.
 *   ws: moe_expert_gateup_workspace(w, act, T, k) bytes (k ignored in the identity form).
 * moe_expert_down writes y_rows[r] = down_e . h[r] from h (FLOAT) or h_codes/h_scales (MXFP4).
 */
moe_status moe_expert_gateup(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k,
                             const void *x, int32_t x_dtype, const int32_t *expert_offsets,
                             const int32_t *sorted_pairs, float *h, uint8_t *h_codes,
                             uint8_t *h_scales, void *ws, size_t ws_bytes, moe_stream stream);
size_t moe_expert_gateup_workspace(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k);
moe_status moe_expert_down(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k,
                           const float *h, const uint8_t *h_codes, const uint8_t *h_scales,
                           const int32_t *expert_offsets, float *y_rows, moe_stream stream);

/*
 * Decode fusion (FLOAT activations; the shared expert fused into the routed launches).
 * (Routed experts plus a shared expert, weighted and summed: rabbit README, design section
 * and architecture table; a step's routed experts in one launch: Rulith Inference README,
 * engine section.)
 * moe_expert_gateup_shared: one launch computes
 *   h[r]        = SwiGLU of the routed expert of row r on its token (as moe_expert_gateup,
 *                 MOE_ACT_FLOAT, with expert_offsets / sorted_pairs), float32 [T*k][d_ff];
 *   h_shared[t] = SwiGLU of `shared` on x[t], float32 [T][shared->d_ff]   (shared != NULL).
 * moe_expert_down_combine: one launch computes the layer output directly
 *   out[t] = sum_{j=0..k-1} topk_w[t][j] * (down_{topk_ids[t][j]} . h[pair_to_row[t*k+j]])
 *            + (shared_gate ? shared_gate[t] : 1) * (shared_down . h_shared[t])
 * in this order, float32 [T][d_model] -- moe_expert_down followed by moe_combine, without
 * the y_rows buffer.  Pairs whose id is outside [0, E) or whose row is -1 contribute 0.
 * shared: one-expert set of the same format and d_model (and, for the down product, d_ff)
 * or NULL.  h and h_shared 16-byte aligned.  A workgroup holds the slots' h rows and a
 * table of 128 partial sums per slot in LDS: with S = k (+1 with a shared expert),
 * S * (4 * roundup(d_ff, 512) + 512) bytes must be <= 150 KiB, else
 * MOE_ERR_UNSUPPORTED.  No workspace.
 */
moe_status moe_expert_gateup_shared(const moe_expert_weights *w, const moe_expert_weights *shared,
                                    int32_t T, int32_t k, const void *x, int32_t x_dtype,
                                    const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                    float *h, float *h_shared, moe_stream stream);
/*
 * moe_router_logits -- the first half of moe_route: the float32 router logits
 *   logits[t][e] = x[t] . w_router[e] (e < E), then logits[t][E] = x[t] . w_shared_gate when
 *   w_shared_gate is given (the shared gate before its sigmoid); [T][E (+1)], row-major.
 *   Same rounding as moe_route (exact bf16 products summed in float64, rounded once).
 *   ws: moe_route_workspace(desc) bytes.  Errors: those of moe_route.
 * moe_topk_gateup_shared -- the rest of moe_route_permute on those logits, then
 *   moe_expert_gateup_shared on its results, as ONE launch: every workgroup of the gate/up
 *   kernel selects the experts from the logits itself (moe_route's selection) before
 *   streaming their weights, so a decode step is moe_router_logits, this call and
 *   moe_expert_down_combine -- three kernels.  (A step's routed experts in one launch, the
 *   host not waiting on the routing: Rulith Inference README, engine section.)
 *   Arguments: desc, logit_bias, select_bias, topk_ids, topk_w, shared_gate, expert_offsets,
 *   sorted_pairs, pair_to_row as for moe_route_permute (has_shared_gate: logits hold the
 *   shared-gate column E, shared_gate is written); w, shared, x (bf16 [T][H]), h, h_shared as
 *   for moe_expert_gateup_shared; desc->E and desc->H must be w's expert count and d_model.
 *   Results: exactly those of moe_route_permute followed by moe_expert_gateup_shared, bit for
 *   bit.  With T <= 4, T*k <= 64, E <= 512 and activation rows that fit in LDS the selection
 *   runs in the gate/up launch; otherwise the route kernel's selection runs first (same
 *   results, one launch more).  No workspace.  Errors: those of the two calls.
 */
moe_status moe_router_logits(const moe_route_desc *desc, const void *x, const void *w_router,
                             const void *w_shared_gate, float *logits, void *ws, size_t ws_bytes, moe_stream stream);
moe_status moe_topk_gateup_shared(const moe_route_desc *desc, const float *logits, const float *logit_bias,
                                  const float *select_bias, int32_t has_shared_gate, const moe_expert_weights *w,
                                  const moe_expert_weights *shared, const void *x, int32_t *topk_ids, float *topk_w,
                                  float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                  int32_t *pair_to_row, float *h, float *h_shared, moe_stream stream);
moe_status moe_expert_down_combine(const moe_expert_weights *w, const moe_expert_weights *shared,
                                   int32_t T, int32_t k, const float *h, const float *h_shared,
                                   const int32_t *topk_ids, const float *topk_w,
                                   const int32_t *pair_to_row, const float *shared_gate, float *out,
                                   moe_stream stream);

/*
 * moe_decode_step -- a whole decode layer step: moe_router_logits, moe_topk_gateup_shared
 * and moe_expert_down_combine as ONE launch ("the routed experts of a step run as one
 * launch" and the host does not wait between its parts: Rulith Inference README, engine
 * section).  The launch runs one workgroup per compute unit, every one resident at once,
 * in three phases that hand over through `sync`: the router logits (rows spread over the
 * workgroups), then the top-k selection in every workgroup with the routed and shared
 * gate/up (the shared expert's weights stream while the logits are awaited), then the
 * down product with the weighted combine (the first down weights are read while the h
 * rows are awaited).
 *   Arguments: desc, x, w_router, w_shared_gate, logit_bias, select_bias as for moe_route
 *   (desc->E and desc->H must be w's expert count and d_model); w, shared as for
 *   moe_expert_gateup_shared / moe_expert_down_combine; the results logits [T][E (+1)],
 *   topk_ids, topk_w, shared_gate (written when w_shared_gate is given), expert_offsets,
 *   sorted_pairs, pair_to_row, h [T*k][d_ff], h_shared [T][d_ff] and out [T][d_model] are
 *   those of the three calls, bit for bit (shared_gate scales the shared term when given).
 *   sync: caller-owned device memory of moe_decode_step_sync_bytes() bytes, zero-filled
 *   once before its first use and then left to the library: word 0 counts the launches
 *   that used it, word 1 is an error word (nonzero after a launch whose hand-off waited
 *   past its bound, tens of milliseconds; that launch's results are undefined), the rest
 *   holds per-workgroup flags and the launch's logits tagged with its count.  A sync buffer serves one stream: launches that use the same
 *   buffer must not overlap, and a launch needs every compute unit for a workgroup, so it
 *   should not share the GPU with another such launch.
 *   The single launch takes MXFP4 weights, 1 <= T <= 4, T*k <= 64, E <= 512, bf16 x rows
 *   that fit in LDS and k (+1) h rows within the down-combine's LDS limit; other shapes
 *   (up to T = 8) run as the three calls, with the same results.  Errors: those of the
 *   three calls, MOE_ERR_INVALID_ARG for T > 8 or a NULL sync.
 */
size_t moe_decode_step_sync_bytes(void);
moe_status moe_decode_step(const moe_route_desc *desc, const void *x, const void *w_router,
                           const void *w_shared_gate, const float *logit_bias, const float *select_bias,
                           const moe_expert_weights *w, const moe_expert_weights *shared, float *logits,
                           int32_t *topk_ids, float *topk_w, float *shared_gate, int32_t *expert_offsets,
                           int32_t *sorted_pairs, int32_t *pair_to_row, float *h, float *h_shared, float *out,
                           uint32_t *sync, moe_stream stream);

/*
 * moe_combine -- atomic-free weighted sum (rabbit README, design section: routed expert
 * outputs summed with their weights, plus the shared expert):
 *   out[t] = sum_{j=0..k-1} topk_w[t][j] * y_rows[pair_to_row[t*k+j]]
 *            + (shared_gate ? shared_gate[t] : 1) * y_shared[t]      (if y_shared != NULL)
 * in this order, float32.  y_rows: [*][d]; y_shared: [T][d] or NULL; out: [T][d].
 */
moe_status moe_combine(int32_t T, int32_t k, int32_t d, const float *y_rows,
                       const int32_t *pair_to_row, const float *topk_w, const float *y_shared,
                       const float *shared_gate, float *out, moe_stream stream);

/*
 * moe_dense_bf16 -- y[t] = W . x[t] (+ residual[t]) with a bf16 weight W [n][kdim],
 * float32 accumulation.  The LatentMoE down/up projections (Kimi K3 article,
 * architecture section: routed experts compute in a narrower latent width).
 * x: [T][kdim] bf16 or float32; residual: float32 [T][n] or NULL; y: float32 [T][n].
 * kdim multiple of 8.
 */
moe_status moe_dense_bf16(int32_t T, int32_t n, int32_t kdim, const void *x, int32_t x_dtype,
                          const void *w, const float *residual, float *y, moe_stream stream);

/*
 * moe_dequant -- decode a weight matrix [n][kdim] to float32 with the conversions of the
 * decode GEMV: each code is decoded unscaled (E2M1 and E4M3 values are exact in bf16 and
 * float32) and multiplied by its scale in float32 -- MXFP4 value E2M1(code) * 2^(s-127)
 * (NaN for s = 255), FP8 value E4M3(code) * scale[n/128][kdim/128].  (The GEMV applies the
 * same scale to each block's partial dot product instead of to each weight.)  codes/scales
 * as in moe_expert_weights for one matrix.  out: float32 [n][kdim].
 * (Formats: rabbit README, architecture table, "native quantization read" row.)
 */
moe_status moe_dequant(int32_t format, int32_t n, int32_t kdim, const uint8_t *codes,
                       const void *scales, float *out, moe_stream stream);

/*
 * moe_dequant_bf16 -- decode an MXFP4 weight matrix [n][kdim] to bf16 with the decoding
 * every matrix-core kernel multiplies (the down-combine of the fused decode, the bf16
 * prefill GEMM, MX activation staging): the gfx950 scaled conversion of each 8-code dword
 * with the block scale 2^(s-127) applied inside the instruction.  E2M1(code) * 2^(s-127) is
 * a bf16 value for every code and scale byte except where it leaves bf16's range.
 * codes: uint8 [n][kdim/2], scales: uint8 E8M0 [n][kdim/32], out: bf16 bits [n][kdim];
 * codes and out 16-byte aligned, kdim a multiple of 32.
 * (The format: rabbit README, opening section and architecture table, OCP MXFP4.)
 */
moe_status moe_dequant_bf16(int32_t n, int32_t kdim, const uint8_t *codes, const uint8_t *scales,
                            uint16_t *out, moe_stream stream);

/*
 * moe_mx_quantize -- OCP MX conversion of rows [rows][cols] (bf16 or float32, cols a
 * multiple of 32) to MXFP4: per 32-block scale byte X+127 with X = floor(log2 amax) - 2
 * clamped to [-127,127] (byte 0 for an all-zero block, 0xFF and zero codes for a block
 * holding NaN or Inf); codes = nearest E2M1 of v/2^X, ties to even, saturating at 6, sign
 * kept.  codes: uint8 [rows][cols/2] (even element in the low nibble); scales: uint8
 * [rows][cols/32].  The activation quantiser of MOE_ACT_MXFP4.
 */
moe_status moe_mx_quantize(int32_t rows, int32_t cols, const void *x, int32_t x_dtype,
                           uint8_t *codes, uint8_t *scales, moe_stream stream);

/* Text of the last error on the calling thread; valid until the next call on it. */
const char *moe_last_error(void);
/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXFP4_ROUTED_EXPERT_MOE_H */

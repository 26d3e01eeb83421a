// Expert FFN entry points: argument checks, workspace layout and kernel selection.
//
// Each expert computes a SwiGLU FFN, h = silu(gate a) * (up a), y = down h (the
// "SituAndMul" activation of the rabbit README source tree, read as SiLU-and-multiply),
// on the rows routed to it.  Small row counts per expert (decode) run on the
// dequant-GEMV kernels; with many rows per expert (prefill) MX-quantised activations run
// on the block-scaled FP4 matrix-core grouped GEMM, and unquantised activations over MXFP4
// weights on the bf16 matrix-core grouped GEMM.
#include "gemv.h"
#include "step_sync.h"

namespace {
constexpr int kRouterDecodeMaxT = 8;   // tokens of a moe_decode_step call
}

namespace moe {

bool mfma_path_wanted(const moe_expert_weights *w, int act, int T, int k, bool routed);
moe_status mfma_gateup_launch(const moe_expert_weights *w, int T, int k, const uint8_t *xq, const uint8_t *xs,
                              const int32_t *offsets, const int32_t *sorted_pairs, int R, float *h,
                              uint8_t *hq, uint8_t *hs, hipStream_t stream);
moe_status mfma_down_launch(const moe_expert_weights *w, const uint8_t *hq, const uint8_t *hs,
                            const int32_t *offsets, int R, float *y, hipStream_t stream);
bool fgemm_wanted(const moe_expert_weights *w, int act, int T);
moe_status fgemm_gateup_launch(const moe_expert_weights *w, int T, int k, const void *x, bool x_f32,
                               const int32_t *offsets, const int32_t *sorted_pairs, int R, float *h,
                               hipStream_t stream);
moe_status fgemm_down_launch(const moe_expert_weights *w, const float *h, const int32_t *offsets, int R, float *y,
                             hipStream_t stream);

namespace {

moe_status validate_weights(const moe_expert_weights *w, int act, const char *fn) {
    MOE_REQUIRE(w != nullptr, "%s: weights descriptor is NULL", fn);
    MOE_REQUIRE(w->format == MOE_W_MXFP4 || w->format == MOE_W_FP8_E4M3_B128, "%s: unknown weight format %d", fn,
                w->format);
    MOE_REQUIRE(w->num_experts >= 1 && w->num_experts <= MOE_MAX_EXPERTS, "%s: num_experts = %d outside [1, %d]", fn,
                w->num_experts, MOE_MAX_EXPERTS);
    MOE_REQUIRE(w->d_model > 0 && w->d_ff > 0, "%s: d_model and d_ff must be positive", fn);
    if (w->format == MOE_W_MXFP4)
        MOE_REQUIRE(w->d_model % 32 == 0 && w->d_ff % 32 == 0,
                    "%s: MXFP4 needs d_model (%d) and d_ff (%d) to be multiples of 32", fn, w->d_model, w->d_ff);
    else
        MOE_REQUIRE(w->d_model % 128 == 0 && w->d_ff % 128 == 0,
                    "%s: FP8 block-128 needs d_model (%d) and d_ff (%d) to be multiples of 128", fn, w->d_model,
                    w->d_ff);
    MOE_REQUIRE(act == MOE_ACT_FLOAT || act == MOE_ACT_MXFP4, "%s: unknown activation mode %d", fn, act);
    MOE_REQUIRE((int64_t)w->num_experts * w->d_ff * w->d_model < ((int64_t)1 << 40),
                "%s: expert stack too large", fn);
    MOE_REQUIRE(w->gate && w->up && w->down && w->gate_s && w->up_s && w->down_s, "%s: NULL weight pointer", fn);
    if (act == MOE_ACT_MXFP4 && w->format != MOE_W_MXFP4) {
        set_error("%s: MX-quantised activations need MXFP4 weights", fn);
        return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

moe_status validate_rows(const moe_expert_weights *w, int T, int k, const int32_t *offsets,
                         const int32_t *sorted_pairs, const char *fn) {
    MOE_REQUIRE(T >= 0, "%s: T = %d < 0", fn, T);
    if (offsets) {
        MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK && k <= w->num_experts, "%s: k = %d outside [1, min(E, %d)]", fn, k,
                    MOE_MAX_TOPK);
        MOE_REQUIRE(sorted_pairs != nullptr || T == 0, "%s: sorted_pairs is NULL", fn);
    } else {
        MOE_REQUIRE(w->num_experts == 1, "%s: expert_offsets == NULL needs exactly one expert (got %d)", fn,
                    w->num_experts);
    }
    const int64_t R = offsets ? (int64_t)T * k : T;
    const int64_t wide = w->d_model > w->d_ff ? w->d_model : w->d_ff;
    MOE_REQUIRE(R * wide < INT32_MAX, "%s: rows x width overflows int32", fn);
    return MOE_OK;
}

inline int rows_of(int T, int k, const int32_t *offsets) { return offsets ? T * k : T; }

struct FfnWs {
    uint8_t *xq = nullptr, *xs = nullptr;   // MX x codes/scales [T][d_model/2], [T][d_model/32]
    float *h = nullptr;                     // [R][d_ff]
    uint8_t *hq = nullptr, *hs = nullptr;   // MX h codes/scales
    size_t bytes = 0;
};

// Workspace layout; `with_h` adds the float32 h buffer, `with_hq` the MX h buffers.
FfnWs ffn_ws_layout(const moe_expert_weights *w, int act, int T, int R, bool with_h, bool with_hq, void *base) {
    FfnWs l;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        unsigned char *p = base ? (unsigned char *)base + off : nullptr;
        off += align_up(bytes, 256);
        return p;
    };
    if (act == MOE_ACT_MXFP4) {
        l.xq = take((size_t)T * w->d_model / 2);
        l.xs = take((size_t)T * w->d_model / 32);
    }
    if (with_h) l.h = (float *)take((size_t)R * w->d_ff * sizeof(float));
    if (with_hq && act == MOE_ACT_MXFP4) {
        l.hq = take((size_t)R * w->d_ff / 2);
        l.hs = take((size_t)R * w->d_ff / 32);
    }
    l.bytes = off;
    return l;
}

GemvParams base_params(const moe_expert_weights *w, int T, int k, const int32_t *offsets,
                       const int32_t *sorted_pairs, int R) {
    GemvParams p = {};
    p.E = w->num_experts;
    p.offsets = offsets;
    p.sorted_pairs = sorted_pairs;
    p.k = k > 0 ? k : 1;
    p.T = T;
    p.R = R;
    return p;
}

moe_status gateup_impl(const moe_expert_weights *w, int act, int T, int k, const void *x, int x_dtype,
                       const int32_t *offsets, const int32_t *sorted_pairs, float *h, uint8_t *hq, uint8_t *hs,
                       const FfnWs &ws, hipStream_t s) {
    const int R = rows_of(T, k, offsets);
    const int fmt = w->format == MOE_W_MXFP4 ? kFmtMXFP4 : kFmtFP8;
    const int slots = offsets ? (w->num_experts < R ? w->num_experts : R) : 1;
    if (act == MOE_ACT_MXFP4) {
        MOE_TRY(mx_quantize_launch(T, w->d_model, x, x_dtype == MOE_DT_F32, ws.xq, ws.xs, s));
        if (mfma_path_wanted(w, act, T, k, offsets != nullptr))
            return mfma_gateup_launch(w, T, k, ws.xq, ws.xs, offsets, sorted_pairs, R, h, hq, hs, s);
    } else if (fgemm_wanted(w, act, T)) {
        return fgemm_gateup_launch(w, T, k, x, x_dtype == MOE_DT_F32, offsets, sorted_pairs, R, h, s);
    }
    GemvParams p = base_params(w, T, k, offsets, sorted_pairs, R);
    p.w[0] = w->gate;
    p.w[1] = w->up;
    p.s[0] = w->gate_s;
    p.s[1] = w->up_s;
    p.N = w->d_ff;
    p.K = w->d_model;
    p.gather = offsets ? 1 : 0;
    p.n_act_rows = T;
    float *hout = h;
    int actk;
    if (act == MOE_ACT_MXFP4) {
        p.act = ws.xq;
        p.act_s = ws.xs;
        actk = kActMX;
        if (!hout) hout = ws.h;
    } else {
        p.act = x;
        actk = x_dtype == MOE_DT_F32 ? kActF32 : kActBF16;
    }
    p.out = hout;
    MOE_TRY(gemv_launch(fmt, actk, true, p, slots, T, s, "moe_expert_gateup"));
    if (act == MOE_ACT_MXFP4) MOE_TRY(mx_quantize_launch(R, w->d_ff, hout, true, hq, hs, s));
    return MOE_OK;
}

moe_status down_impl(const moe_expert_weights *w, int act, int T, int k, const float *h, const uint8_t *hq,
                     const uint8_t *hs, const int32_t *offsets, float *y, hipStream_t s) {
    const int R = rows_of(T, k, offsets);
    const int fmt = w->format == MOE_W_MXFP4 ? kFmtMXFP4 : kFmtFP8;
    const int slots = offsets ? (w->num_experts < R ? w->num_experts : R) : 1;
    if (act == MOE_ACT_MXFP4 && mfma_path_wanted(w, act, T, k, offsets != nullptr))
        return mfma_down_launch(w, hq, hs, offsets, R, y, s);
    if (act == MOE_ACT_FLOAT && fgemm_wanted(w, act, T)) return fgemm_down_launch(w, h, offsets, R, y, s);
    GemvParams p = base_params(w, T, k, offsets, nullptr, R);
    p.w[0] = w->down;
    p.s[0] = w->down_s;
    p.N = w->d_model;
    p.K = w->d_ff;
    p.gather = 0;
    p.n_act_rows = R;
    p.out = y;
    int actk;
    if (act == MOE_ACT_MXFP4) {
        p.act = hq;
        p.act_s = hs;
        actk = kActMX;
    } else {
        p.act = h;
        actk = kActF32;
    }
    return gemv_launch(fmt, actk, false, p, slots, T, s, "moe_expert_down");
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_expert_gateup_workspace(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k) {
    if (!w || T <= 0) return 0;
    if (act != MOE_ACT_MXFP4) return 0;
    const int R = T * (k > 0 ? k : 1);
    return ffn_ws_layout(w, act, T, R, true, false, nullptr).bytes;
}

extern "C" size_t moe_expert_ffn_workspace(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k) {
    if (!w || T <= 0) return 0;
    const int R = T * (k > 0 ? k : 1);
    return ffn_ws_layout(w, act, T, R, true, true, nullptr).bytes;
}

extern "C" moe_status moe_expert_gateup(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k,
                                        const void *x, int32_t x_dtype, const int32_t *expert_offsets,
                                        const int32_t *sorted_pairs, float *h, uint8_t *h_codes,
                                        uint8_t *h_scales, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_weights(w, act, "moe_expert_gateup"));
    MOE_TRY(validate_rows(w, T, k, expert_offsets, sorted_pairs, "moe_expert_gateup"));
    MOE_REQUIRE(x_dtype == MOE_DT_BF16 || x_dtype == MOE_DT_F32, "moe_expert_gateup: unknown x_dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(x != nullptr, "moe_expert_gateup: NULL x");
    if (act == MOE_ACT_FLOAT)
        MOE_REQUIRE(h != nullptr, "moe_expert_gateup: NULL h (required with MOE_ACT_FLOAT)");
    else
        MOE_REQUIRE(h_codes && h_scales, "moe_expert_gateup: NULL h_codes or h_scales (required with MOE_ACT_MXFP4)");
    const int R = rows_of(T, k, expert_offsets);
    const size_t need = moe_expert_gateup_workspace(w, act, T, expert_offsets ? k : 1);
    if (need && (!ws || ws_bytes < need)) {
        set_error("moe_expert_gateup: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        return MOE_ERR_WORKSPACE;
    }
    FfnWs l = ffn_ws_layout(w, act, T, R, true, false, ws);
    return gateup_impl(w, act, T, k, x, x_dtype, expert_offsets, sorted_pairs, h, h_codes, h_scales, l,
                       (hipStream_t)stream);
}

extern "C" moe_status moe_expert_down(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k, const float *h,
                                      const uint8_t *h_codes, const uint8_t *h_scales, const int32_t *expert_offsets,
                                      float *y_rows, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_weights(w, act, "moe_expert_down"));
    MOE_TRY(validate_rows(w, T, k, expert_offsets, (const int32_t *)1, "moe_expert_down"));
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(y_rows != nullptr, "moe_expert_down: NULL y_rows");
    if (act == MOE_ACT_FLOAT)
        MOE_REQUIRE(h != nullptr, "moe_expert_down: NULL h (required with MOE_ACT_FLOAT)");
    else
        MOE_REQUIRE(h_codes && h_scales, "moe_expert_down: NULL h_codes or h_scales (required with MOE_ACT_MXFP4)");
    return down_impl(w, act, T, k, h, h_codes, h_scales, expert_offsets, y_rows, (hipStream_t)stream);
}

extern "C" moe_status moe_expert_ffn(const moe_expert_weights *w, int32_t act, int32_t T, int32_t k, const void *x,
                                     int32_t x_dtype, const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                     float *y_rows, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_weights(w, act, "moe_expert_ffn"));
    MOE_TRY(validate_rows(w, T, k, expert_offsets, sorted_pairs, "moe_expert_ffn"));
    MOE_REQUIRE(x_dtype == MOE_DT_BF16 || x_dtype == MOE_DT_F32, "moe_expert_ffn: unknown x_dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(x && y_rows, "moe_expert_ffn: NULL x or y_rows");
    const int kk = expert_offsets ? k : 1;
    const int R = rows_of(T, k, expert_offsets);
    const size_t need = moe_expert_ffn_workspace(w, act, T, kk);
    if (!ws || ws_bytes < need) {
        set_error("moe_expert_ffn: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        return MOE_ERR_WORKSPACE;
    }
    FfnWs l = ffn_ws_layout(w, act, T, R, true, true, ws);
    hipStream_t s = (hipStream_t)stream;
    // MX mode hands h to the down product as codes only; float32 h is an intermediate of
    // the GEMV form alone (which takes it from the workspace itself).
    float *h = act == MOE_ACT_MXFP4 ? nullptr : l.h;
    MOE_TRY(gateup_impl(w, act, T, k, x, x_dtype, expert_offsets, sorted_pairs, h, l.hq, l.hs, l, s));
    return down_impl(w, act, T, k, l.h, l.hq, l.hs, expert_offsets, y_rows, s);
}

// ------------------------------------------------------------------ decode fusion

namespace moe {
namespace {

moe_status validate_shared(const moe_expert_weights *w, const moe_expert_weights *sh, const char *fn) {
    if (!sh) return MOE_OK;
    MOE_TRY(validate_weights(sh, MOE_ACT_FLOAT, fn));
    MOE_REQUIRE(sh->num_experts == 1, "%s: the shared expert set must hold one expert (got %d)", fn, sh->num_experts);
    MOE_REQUIRE(sh->format == w->format && sh->d_model == w->d_model,
                "%s: the shared expert must have the routed experts' format and d_model", fn);
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_expert_gateup_shared(const moe_expert_weights *w, const moe_expert_weights *shared,
                                               int32_t T, int32_t k, const void *x, int32_t x_dtype,
                                               const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                               float *h, float *h_shared, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_weights(w, MOE_ACT_FLOAT, "moe_expert_gateup_shared"));
    MOE_TRY(validate_shared(w, shared, "moe_expert_gateup_shared"));
    MOE_REQUIRE(expert_offsets != nullptr, "moe_expert_gateup_shared: NULL expert_offsets");
    MOE_TRY(validate_rows(w, T, k, expert_offsets, sorted_pairs, "moe_expert_gateup_shared"));
    MOE_REQUIRE(x_dtype == MOE_DT_BF16 || x_dtype == MOE_DT_F32, "moe_expert_gateup_shared: unknown x_dtype %d",
                x_dtype);
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(x && h, "moe_expert_gateup_shared: NULL x or h");
    MOE_REQUIRE(!shared || h_shared, "moe_expert_gateup_shared: NULL h_shared with a shared expert");
    if (shared) MOE_REQUIRE((int64_t)T * shared->d_ff < INT32_MAX, "moe_expert_gateup_shared: sizes overflow int32");
    const int R = T * k;
    const int fmt = w->format == MOE_W_MXFP4 ? kFmtMXFP4 : kFmtFP8;
    const int slots = w->num_experts < R ? w->num_experts : R;
    GemvParams p = base_params(w, T, k, expert_offsets, sorted_pairs, R);
    p.w[0] = w->gate;
    p.w[1] = w->up;
    p.s[0] = w->gate_s;
    p.s[1] = w->up_s;
    p.N = w->d_ff;
    p.K = w->d_model;
    p.gather = 1;
    p.n_act_rows = T;
    p.act = x;
    p.out = h;
    if (shared) {
        p.shared_slot = slots;
        p.sw[0] = shared->gate;
        p.sw[1] = shared->up;
        p.ss[0] = shared->gate_s;
        p.ss[1] = shared->up_s;
        p.sN = shared->d_ff;
        p.sout = h_shared;
    }
    return gemv_launch(fmt, x_dtype == MOE_DT_F32 ? kActF32 : kActBF16, true, p, slots + (shared ? 1 : 0), T,
                       (hipStream_t)stream, "moe_expert_gateup_shared");
}

// Parameters of the gate/up launch that routes in its prologue (moe_topk_gateup_shared).
static GemvParams topk_gateup_params(const moe_route_desc *d, const float *logits, const float *logit_bias,
                                     const float *select_bias, int32_t has_shared_gate, const moe_expert_weights *w,
                                     const moe_expert_weights *shared, const void *x, int32_t *topk_ids,
                                     float *topk_w, float *shared_gate, int32_t *expert_offsets,
                                     int32_t *sorted_pairs, int32_t *pair_to_row, float *h, float *h_shared) {
    const int T = d->T, k = d->k, R = T * k;
    const int slots = w->num_experts < R ? w->num_experts : R;
    GemvParams p = base_params(w, T, k, nullptr, nullptr, R);
    p.w[0] = w->gate;
    p.w[1] = w->up;
    p.s[0] = w->gate_s;
    p.s[1] = w->up_s;
    p.N = w->d_ff;
    p.K = w->d_model;
    p.gather = 1;
    p.n_act_rows = T;
    p.act = x;
    p.out = h;
    if (shared) {
        p.shared_slot = slots;
        p.sw[0] = shared->gate;
        p.sw[1] = shared->up;
        p.ss[0] = shared->gate_s;
        p.ss[1] = shared->up_s;
        p.sN = shared->d_ff;
        p.sout = h_shared;
    }
    RouteArgs &ra = p.route;
    ra.logits = logits;
    ra.rows = d->E + (has_shared_gate ? 1 : 0);
    ra.score = d->score;
    ra.renorm = d->renormalize;
    ra.scaling = d->routed_scaling;
    ra.lbias = logit_bias;
    ra.sbias = select_bias;
    ra.has_sg = has_shared_gate ? 1 : 0;
    ra.n_group = d->n_group > 1 ? d->n_group : 1;
    ra.topk_group = d->n_group > 1 ? d->topk_group : 1;
    ra.ids = topk_ids;
    ra.tw = topk_w;
    ra.sg = shared_gate;
    ra.offsets = expert_offsets;
    ra.sorted = sorted_pairs;
    ra.p2r = pair_to_row;
    return p;
}

extern "C" moe_status moe_topk_gateup_shared(const moe_route_desc *d, const float *logits, const float *logit_bias,
                                             const float *select_bias, int32_t has_shared_gate,
                                             const moe_expert_weights *w, const moe_expert_weights *shared,
                                             const void *x, int32_t *topk_ids, float *topk_w, float *shared_gate,
                                             int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_to_row,
                                             float *h, float *h_shared, moe_stream stream) {
    clear_error();
    const char *fn = "moe_topk_gateup_shared";
    MOE_TRY(check_route_desc(d));
    MOE_TRY(validate_weights(w, MOE_ACT_FLOAT, fn));
    MOE_TRY(validate_shared(w, shared, fn));
    MOE_REQUIRE(d->E == w->num_experts && d->H == w->d_model,
                "%s: the router's E = %d and H = %d must be the experts' count (%d) and d_model (%d)", fn, d->E, d->H,
                w->num_experts, w->d_model);
    MOE_REQUIRE(!(select_bias && d->score != MOE_SCORE_SIGMOID), "%s: select_bias is only defined for MOE_SCORE_SIGMOID",
                fn);
    MOE_REQUIRE(expert_offsets && sorted_pairs && pair_to_row, "%s: NULL expert_offsets, sorted_pairs or pair_to_row",
                fn);
    MOE_REQUIRE((int64_t)d->T * d->k < INT32_MAX && (int64_t)d->T * w->d_ff < INT32_MAX, "%s: sizes overflow int32", fn);
    if (d->T == 0) return moe_permute(0, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0,
                                      stream);
    MOE_REQUIRE(logits && x && topk_ids && topk_w && h, "%s: NULL logits, x, topk_ids, topk_w or h", fn);
    MOE_REQUIRE(!has_shared_gate || shared_gate, "%s: NULL shared_gate with has_shared_gate", fn);
    MOE_REQUIRE(!shared || h_shared, "%s: NULL h_shared with a shared expert", fn);
    hipStream_t s = (hipStream_t)stream;
    const int T = d->T, k = d->k, R = T * k;
    const int fmt = w->format == MOE_W_MXFP4 ? kFmtMXFP4 : kFmtFP8;
    const int slots = w->num_experts < R ? w->num_experts : R;
    const GemvParams p = topk_gateup_params(d, logits, logit_bias, select_bias, has_shared_gate, w, shared, x, topk_ids,
                                            topk_w, shared_gate, expert_offsets, sorted_pairs, pair_to_row, h,
                                            h_shared);
    moe_status st = MOE_OK;
    if (gemv_route_launch(fmt, kActBF16, p, slots + (shared ? 1 : 0), s, &st)) return st;
    // shapes the routing-in-the-prologue form does not take: the route kernel's selection,
    // then the gate/up launch on its permutation
    MOE_TRY(route_select_step(d, logits, logit_bias, select_bias, has_shared_gate != 0, topk_ids, topk_w, shared_gate,
                              expert_offsets, sorted_pairs, pair_to_row, s));
    return moe_expert_gateup_shared(w, shared, T, k, x, MOE_DT_BF16, expert_offsets, sorted_pairs, h, h_shared,
                                    stream);
}

// Parameters of the down-combine launch (moe_expert_down_combine).
static DownCombineParams down_combine_params(const moe_expert_weights *w, const moe_expert_weights *shared, int32_t T,
                                             int32_t k, const float *h, const float *h_shared,
                                             const int32_t *topk_ids, const float *topk_w,
                                             const int32_t *pair_to_row, const float *shared_gate, float *out) {
    DownCombineParams p = {};
    p.w = w->down;
    p.s = w->down_s;
    p.sw = shared ? shared->down : nullptr;
    p.ss = shared ? shared->down_s : nullptr;
    p.E = w->num_experts;
    p.N = w->d_model;
    p.I = w->d_ff;
    p.h = h;
    p.hs = h_shared;
    p.ids = topk_ids;
    p.tw = topk_w;
    p.p2r = pair_to_row;
    p.sg = shared ? shared_gate : nullptr;
    p.T = T;
    p.k = k;
    p.R = T * k;
    p.out = out;
    return p;
}

extern "C" moe_status moe_expert_down_combine(const moe_expert_weights *w, const moe_expert_weights *shared,
                                              int32_t T, int32_t k, const float *h, const float *h_shared,
                                              const int32_t *topk_ids, const float *topk_w,
                                              const int32_t *pair_to_row, const float *shared_gate, float *out,
                                              moe_stream stream) {
    clear_error();
    MOE_TRY(validate_weights(w, MOE_ACT_FLOAT, "moe_expert_down_combine"));
    MOE_TRY(validate_shared(w, shared, "moe_expert_down_combine"));
    MOE_REQUIRE(T >= 0, "moe_expert_down_combine: T = %d < 0", T);
    MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK && k <= w->num_experts,
                "moe_expert_down_combine: k = %d outside [1, min(E, %d)]", k, MOE_MAX_TOPK);
    MOE_REQUIRE((int64_t)T * k * w->d_ff < INT32_MAX && (int64_t)T * w->d_model < INT32_MAX,
                "moe_expert_down_combine: sizes overflow int32");
    if (shared)
        MOE_REQUIRE(shared->d_ff == w->d_ff, "moe_expert_down_combine: the shared expert's d_ff (%d) must equal d_ff (%d)",
                    shared->d_ff, w->d_ff);
    if (down_combine_lds(k, shared != nullptr, w->d_ff) > 150 * 1024) {
        set_error("moe_expert_down_combine: %d rows of d_ff = %d and the output table do not fit in LDS",
                  k + (shared ? 1 : 0), w->d_ff);
        return MOE_ERR_UNSUPPORTED;
    }
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(h && topk_ids && topk_w && pair_to_row && out, "moe_expert_down_combine: NULL pointer argument");
    MOE_REQUIRE(!shared || h_shared, "moe_expert_down_combine: NULL h_shared with a shared expert");
    MOE_REQUIRE((((uintptr_t)h | (uintptr_t)h_shared) & 15) == 0, "moe_expert_down_combine: h and h_shared must be "
                "16-byte aligned");
    const DownCombineParams p = down_combine_params(w, shared, T, k, h, h_shared, topk_ids, topk_w, pair_to_row,
                                                    shared_gate, out);
    return down_combine_launch(w->format == MOE_W_MXFP4 ? kFmtMXFP4 : kFmtFP8, p, (hipStream_t)stream);
}

extern "C" size_t moe_decode_step_sync_bytes(void) { return (size_t)kSyncWords * sizeof(uint32_t); }

extern "C" moe_status moe_decode_step(const moe_route_desc *d, const void *x, const void *w_router,
                                      const void *w_shared_gate, const float *logit_bias, const float *select_bias,
                                      const moe_expert_weights *w, const moe_expert_weights *shared, float *logits,
                                      int32_t *topk_ids, float *topk_w, float *shared_gate, int32_t *expert_offsets,
                                      int32_t *sorted_pairs, int32_t *pair_to_row, float *h, float *h_shared,
                                      float *out, uint32_t *sync, moe_stream stream) {
    clear_error();
    const char *fn = "moe_decode_step";
    MOE_TRY(check_route_desc(d));
    MOE_TRY(validate_weights(w, MOE_ACT_FLOAT, fn));
    MOE_TRY(validate_shared(w, shared, fn));
    MOE_REQUIRE(d->E == w->num_experts && d->H == w->d_model,
                "%s: the router's E = %d and H = %d must be the experts' count (%d) and d_model (%d)", fn, d->E, d->H,
                w->num_experts, w->d_model);
    MOE_REQUIRE(d->T <= kRouterDecodeMaxT, "%s: T = %d above %d (a decode step)", fn, d->T, kRouterDecodeMaxT);
    MOE_REQUIRE(!(select_bias && d->score != MOE_SCORE_SIGMOID), "%s: select_bias is only defined for MOE_SCORE_SIGMOID",
                fn);
    MOE_REQUIRE(expert_offsets && sorted_pairs && pair_to_row, "%s: NULL expert_offsets, sorted_pairs or pair_to_row",
                fn);
    if (shared)
        MOE_REQUIRE(shared->d_ff == w->d_ff, "%s: the shared expert's d_ff (%d) must equal d_ff (%d)", fn,
                    shared->d_ff, w->d_ff);
    if (down_combine_lds(d->k, shared != nullptr, w->d_ff) > 150 * 1024) {
        set_error("%s: %d rows of d_ff = %d and the output table do not fit in LDS", fn, d->k + (shared ? 1 : 0),
                  w->d_ff);
        return MOE_ERR_UNSUPPORTED;
    }
    if (d->T == 0) return moe_permute(0, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0,
                                      stream);
    MOE_REQUIRE(x && w_router && logits && topk_ids && topk_w && h && out && sync,
                "%s: NULL x, w_router, logits, topk_ids, topk_w, h, out or sync", fn);
    MOE_REQUIRE(!w_shared_gate || shared_gate, "%s: NULL shared_gate with w_shared_gate", fn);
    MOE_REQUIRE(!shared || h_shared, "%s: NULL h_shared with a shared expert", fn);
    MOE_REQUIRE((((uintptr_t)h | (uintptr_t)h_shared) & 15) == 0, "%s: h and h_shared must be 16-byte aligned", fn);
    MOE_REQUIRE(((uintptr_t)sync & 3) == 0, "%s: sync must be 4-byte aligned", fn);
    hipStream_t s = (hipStream_t)stream;
    const int has_sg = w_shared_gate ? 1 : 0;
    StepParams sp = {};
    sp.gu = topk_gateup_params(d, logits, logit_bias, select_bias, has_sg, w, shared, x, topk_ids, topk_w, shared_gate,
                               expert_offsets, sorted_pairs, pair_to_row, h, h_shared);
    sp.dc = down_combine_params(w, shared, d->T, d->k, h, h_shared, topk_ids, topk_w, pair_to_row,
                                has_sg ? shared_gate : nullptr, out);
    sp.x = (const uint16_t *)x;
    sp.wr = (const uint16_t *)w_router;
    sp.wsg = (const uint16_t *)w_shared_gate;
    sp.T = d->T;
    sp.H = d->H;
    sp.E = d->E;
    sp.rows = d->E + has_sg;
    sp.logits = logits;
    sp.sync = sync;
    moe_status st = MOE_OK;
    if (w->format == MOE_W_MXFP4 && decode_step_launch(sp, s, &st)) return st;
    // shapes the single launch does not take: the three-call form, same results
    MOE_TRY(router_logits_small(d, x, w_router, w_shared_gate, logits, s));
    MOE_TRY(moe_topk_gateup_shared(d, logits, logit_bias, select_bias, has_sg, w, shared, x, topk_ids, topk_w,
                                   shared_gate, expert_offsets, sorted_pairs, pair_to_row, h, h_shared, stream));
    return moe_expert_down_combine(w, shared, d->T, d->k, h, h_shared, topk_ids, topk_w, pair_to_row,
                                   has_sg ? shared_gate : nullptr, out, stream);
}

// Router: logits, scoring, top-k and renormalisation.
//
// Routing schemes of the pages: "softmax top-10 of 512 + gated shared expert"
// (Qwen3.8-Max) and "noaux_tc sigmoid" (GLM-5.2) -- rabbit README, architecture table,
// "MoE routing" row.  The logit of (t, e) is the float32 rounding of the exact dot
// product of two bf16 vectors: bf16 x bf16 products are exact in float64 and the sum
// is accumulated in float64, then rounded once.  Scoring, top-k and the weights run in
// float64; only the final weights are rounded to float32.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <mutex>

#include "common.h"
#include "router_row.h"
#include "topk.h"

namespace moe {
namespace {

// A workgroup computes the dot products of one weight row (expert e < E, or the shared
// gate row e == E) with up to kRouterTB tokens; wave w covers the w-th quarter of H
// (router_quarter), so a row is read with four waves' worth of loads in flight, and the
// quarters are added in order.
__global__ __launch_bounds__(64 * kRouterWaves) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                                         const uint16_t *__restrict__ wr,
                                                                         const uint16_t *__restrict__ wsg,
                                                                         int T, int H, int E, int rows,
                                                                         float *__restrict__ logits) {
    __shared__ double part[kRouterWaves][kRouterTB];
    const int row = blockIdx.x;
    const uint16_t *w = row < E ? wr + (size_t)row * H : wsg;
    const int t0 = blockIdx.y * kRouterTB;
    const int nt = min(kRouterTB, T - t0);
    const int lane = lane_id(), wave = wave_id();
    double s[kRouterTB];
    router_quarter(x, w, t0, nt, H, wave, s);
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) {
        if (t >= nt) break;
        if (lane == 0) part[wave][t] = s[t];
    }
    __syncthreads();
    if (threadIdx.x < nt) logits[(size_t)(t0 + threadIdx.x) * rows + row] = router_finish(part, threadIdx.x);
}

// Many tokens: a tiled float64 product on the matrix cores.  A workgroup owns 128 tokens x
// 64 rows and one of kRouterKS slices of H; bf16 tiles are converted once to float64 into
// LDS (k-major).  Wave w multiplies tokens 32w .. 32w+31 by the 64 rows with
// v_mfma_f64_16x16x4_f64 (lane l supplies A[l%16][l/16] and B[l/16][l%16]; it receives
// C[l/16 + 4i][l%16]); the products of two bf16 values are exact in float64 and the sums
// are float64.  The next stage's values are loaded while the current one is multiplied.
// The slices' partial sums go to the workspace and router_reduce_kernel adds them in a
// fixed order and rounds once to float32 -- the same logits as the one-wave form, up to
// float64 rounding.
constexpr int kRouterKS = 16;   // K slices
constexpr int kRtTok = 128;     // tokens per tile
constexpr int kRtRow = 64;      // rows per tile
constexpr int kRtKC = 32;       // bf16 values per stage
constexpr int kRtThin = 16;     // row tiles with at most this many rows use plain dot products

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ wr,
                                                              const uint16_t *__restrict__ wsg, int T, int H,
                                                              int E, int rows, double *__restrict__ partial) {
    __shared__ __align__(16) double xs[kRtKC][kRtTok];
    __shared__ __align__(16) double wsm[kRtKC][kRtRow];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * kRtTok, r0 = blockIdx.x * kRtRow;
    const int ks = blockIdx.z;
    const int hs = H / kRouterKS;                      // H % (32 * kRouterKS) is checked on the host
    const int h0 = ks * hs, h1 = h0 + hs;
    auto wrow_of = [&](int r) { return r < E ? wr + (size_t)r * H : wsg; };

    // A tile with few rows (the shared-gate row after a whole number of row tiles, or a
    // small E): each (token, row) pair of the tile is one thread's plain dot product over the
    // slice, in the same order as the tiled form.
    if (rows - r0 <= kRtThin) {
        const int nr = rows - r0;
        for (int i = tid; i < kRtTok * nr; i += 256) {
            const int t = t0 + i / nr, r = r0 + i % nr;
            if (t >= T) continue;
            const uint16_t *xr = x + (size_t)t * H, *wrr = wrow_of(r);
            double s = 0.0;
            for (int h = h0; h < h1; h += 8) {
                const u32x4 xv = *(const u32x4 *)(xr + h), wv = *(const u32x4 *)(wrr + h);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 fx = bf16x2_to_f32x2(xv[q]), fw = bf16x2_to_f32x2(wv[q]);
                    s = fma((double)fx.x, (double)fw.x, s);
                    s = fma((double)fx.y, (double)fw.y, s);
                }
            }
            partial[((size_t)ks * T + t) * rows + r] = s;
        }
        return;
    }

    const int lane = lane_id(), wave = wave_id();
    const int lr = lane & 15, lk = lane >> 4;          // MFMA operand row/column, K index
    // staging (kRtKC = 32 values a stage): x thread -> (token tid/2, 16 values at (tid&1)*16);
    // w thread -> (row tid/4, 8 values at (tid&3)*8)
    const int lt = tid >> 1, lh = (tid & 1) * 16;
    const int lw = tid >> 2, lq = (tid & 3) * 8;
    const int tt = min(t0 + lt, T - 1), rr = min(r0 + lw, rows - 1);
    const bool tok_ok = t0 + lt < T, row_ok = r0 + lw < rows;
    const uint16_t *xrow = x + (size_t)tt * H;
    const uint16_t *wrow = wrow_of(rr);
    f64x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    u32x4 xv0 = *(const u32x4 *)(xrow + h0 + lh), xv1 = *(const u32x4 *)(xrow + h0 + lh + 8);
    u32x4 wv = __builtin_nontemporal_load((const u32x4 *)(wrow + h0 + lq));
    for (int h = h0; h < h1; h += kRtKC) {
        lds_barrier();                                 // the previous stage is consumed
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x2 f0 = bf16x2_to_f32x2(xv0[q]), f1 = bf16x2_to_f32x2(xv1[q]);
            xs[lh + 2 * q][lt] = tok_ok ? (double)f0.x : 0.0;
            xs[lh + 2 * q + 1][lt] = tok_ok ? (double)f0.y : 0.0;
            xs[lh + 8 + 2 * q][lt] = tok_ok ? (double)f1.x : 0.0;
            xs[lh + 8 + 2 * q + 1][lt] = tok_ok ? (double)f1.y : 0.0;
            const f32x2 fw = bf16x2_to_f32x2(wv[q]);
            wsm[lq + 2 * q][lw] = row_ok ? (double)fw.x : 0.0;
            wsm[lq + 2 * q + 1][lw] = row_ok ? (double)fw.y : 0.0;
        }
        const int hn = min(h + kRtKC, h1 - kRtKC);     // (the last stage reloads itself, unused)
        xv0 = *(const u32x4 *)(xrow + hn + lh);
        xv1 = *(const u32x4 *)(xrow + hn + lh + 8);
        wv = __builtin_nontemporal_load((const u32x4 *)(wrow + hn + lq));
        lds_barrier();                                 // (the next stage's loads stay in flight)
#pragma unroll
        for (int k0 = 0; k0 < kRtKC; k0 += 4) {
            double a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = xs[k0 + lk][32 * wave + 16 * i + lr];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = wsm[k0 + lk][16 * j + lr];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = t0 + 32 * wave + 16 * i + lk + 4 * v;
            if (t >= T) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 16 * j + lr;
                if (r < rows) partial[((size_t)ks * T + t) * rows + r] = acc[i][j][v];
            }
        }
}

__global__ __launch_bounds__(256) void router_reduce_kernel(const double *__restrict__ partial, int n,
                                                            float *__restrict__ logits) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double s = 0.0;
#pragma unroll
    for (int ks = 0; ks < kRouterKS; ++ks) s += partial[(size_t)ks * n + i];
    logits[i] = (float)s;
}

bool router_tiled(const moe_route_desc *d) { return d->T >= 32 && d->H % (32 * kRouterKS) == 0; }

// One wave per token (topk_select).
// PERM: one workgroup holds every token (T <= 4, T*k <= 64) and also writes the token ->
// expert permutation of the selected ids, as moe_permute would.
template <int NK, bool PERM>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int rows,
                                                   int T, int E, int k, int score, int renorm,
                                                   float scaling, const float *__restrict__ lbias,
                                                   const float *__restrict__ sbias, int has_sg,
                                                   int32_t *__restrict__ ids, float *__restrict__ w,
                                                   float *__restrict__ sg, int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ sorted, int32_t *__restrict__ p2r,
                                                   int n_group, int topk_group) {
    __shared__ int sid[PERM ? 64 : 1];
    extern __shared__ double s_gkey[];      // [4 waves][E] selection keys, group-limited form only
    const int t = blockIdx.x * 4 + wave_id();
    if (!PERM && t >= T) return;
    const int lane = lane_id();
    if (t < T) {
        const TopkLane r = topk_select<NK>(logits + (size_t)t * rows, E, k, score, renorm, scaling, lbias, sbias,
                                           has_sg, s_gkey + wave_id() * E, n_group, topk_group);
        if (lane < k) {
            ids[(size_t)t * k + lane] = r.e;
            w[(size_t)t * k + lane] = r.w;
            if constexpr (PERM) sid[t * k + lane] = r.e;        // -1 when fewer than k keys compare
        }
        if (has_sg && lane == 0) sg[t] = r.sg;
    }
    if constexpr (PERM) {
        lds_barrier();           // sid is in LDS; the id and weight stores need not land first
        small_permutation(sid, T * k, E, offsets, sorted, p2r, threadIdx.x, blockDim.x);
    }
}

moe_status validate_route(const moe_route_desc *d) {
    MOE_REQUIRE(d != nullptr, "moe_route: desc is NULL");
    MOE_REQUIRE(d->T >= 0, "moe_route: T = %d < 0", d->T);
    MOE_REQUIRE(d->H > 0 && d->H % 32 == 0, "moe_route: H = %d must be a positive multiple of 32", d->H);
    MOE_REQUIRE(d->E >= 1 && d->E <= MOE_MAX_EXPERTS, "moe_route: E = %d outside [1, %d]", d->E,
                MOE_MAX_EXPERTS);
    MOE_REQUIRE(d->k >= 1 && d->k <= MOE_MAX_TOPK && d->k <= d->E,
                "moe_route: k = %d outside [1, min(E, %d)]", d->k, MOE_MAX_TOPK);
    MOE_REQUIRE(d->score == MOE_SCORE_SOFTMAX || d->score == MOE_SCORE_SIGMOID,
                "moe_route: unknown score %d", d->score);
    MOE_REQUIRE((int64_t)d->T * (d->E + 1) < INT32_MAX && (int64_t)d->T * d->H < INT32_MAX,
                "moe_route: sizes overflow int32");
    if (d->n_group > 1) {
        const int ng = d->n_group, gs = d->E / ng;
        MOE_REQUIRE(ng <= 64 && d->E % ng == 0, "moe_route: n_group = %d must divide E = %d and be <= 64", ng, d->E);
        MOE_REQUIRE(d->score != MOE_SCORE_SIGMOID || gs >= 2,
                    "moe_route: sigmoid group scores need at least 2 experts per group (E / n_group = %d)", gs);
        MOE_REQUIRE(d->topk_group >= 1 && d->topk_group <= ng && (int64_t)d->topk_group * gs >= d->k,
                    "moe_route: topk_group = %d must be in [1, n_group] and keep at least k experts", d->topk_group);
    } else {
        MOE_REQUIRE(d->n_group >= 0, "moe_route: n_group = %d < 0", d->n_group);
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {

template <bool PERM>
moe_status launch_topk_t(const moe_route_desc *d, const float *logits, int rows, const float *lb, const float *sb,
                         bool has_sg, int32_t *ids, float *w, float *sg, int32_t *offs, int32_t *sorted,
                         int32_t *p2r, hipStream_t s) {
    auto topk = d->E <= 256 ? topk_kernel<4, PERM> : d->E <= 512 ? topk_kernel<8, PERM>
              : d->E <= 1024 ? topk_kernel<16, PERM> : topk_kernel<32, PERM>;
    const int tb = (d->T < 4 && !PERM) ? 64 * d->T : 256;   // the permutation uses every thread
    const int ng = d->n_group > 1 ? d->n_group : 1;
    const size_t lds = ng > 1 ? (size_t)(tb / 64) * d->E * sizeof(double) : 0;
    hipLaunchKernelGGL(topk, dim3((d->T + 3) / 4), dim3(tb), lds, s, logits, rows, d->T, d->E, d->k, d->score,
                       d->renormalize, d->routed_scaling, lb, sb, has_sg ? 1 : 0, ids, w, sg, offs, sorted, p2r, ng,
                       ng > 1 ? d->topk_group : 1);
    return launch_check(PERM ? "moe_route_permute: topk_kernel" : "moe_route: topk_kernel");
}

moe_status launch_topk(const moe_route_desc *d, const float *logits, int rows, const float *lb, const float *sb,
                       bool has_sg, int32_t *ids, float *w, float *sg, int32_t *offs, int32_t *sorted, int32_t *p2r,
                       hipStream_t s) {
    if (offs) return launch_topk_t<true>(d, logits, rows, lb, sb, has_sg, ids, w, sg, offs, sorted, p2r, s);
    return launch_topk_t<false>(d, logits, rows, lb, sb, has_sg, ids, w, sg, nullptr, nullptr, nullptr, s);
}

}  // namespace

extern "C" size_t moe_route_workspace(const moe_route_desc *d) {
    if (!d || d->T <= 0 || d->E <= 0) return 0;
    size_t b = align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256);
    if (d->H % 32 == 0 && router_tiled(d)) b += (size_t)kRouterKS * d->T * (d->E + 1) * sizeof(double);
    return b;
}

namespace {

// Checks the routing arguments and enqueues the logits (router_logits_kernel, or the tiled
// product and its reduction) into the workspace.
// Enqueues the float32 logits [T][E (+1 for the shared-gate row)] (router_logits_kernel, or
// the tiled product into `partial` and its reduction).
moe_status enqueue_logits(const moe_route_desc *d, const void *x, const void *w_router, const void *w_shared_gate,
                          float *logits, double *partial, hipStream_t s) {
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    if (router_tiled(d)) {
        dim3 gt((rows + kRtRow - 1) / kRtRow, (d->T + kRtTok - 1) / kRtTok, kRouterKS);
        hipLaunchKernelGGL(router_tiled_kernel, gt, dim3(256), 0, s, (const uint16_t *)x, (const uint16_t *)w_router,
                           (const uint16_t *)w_shared_gate, d->T, d->H, d->E, rows, partial);
        MOE_TRY(launch_check("moe_route: router_tiled_kernel"));
        const int n = d->T * rows;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, partial, n, logits);
        return launch_check("moe_route: router_reduce_kernel");
    }
    dim3 g1(rows, (d->T + kRouterTB - 1) / kRouterTB);
    hipLaunchKernelGGL(router_logits_kernel, g1, dim3(64 * kRouterWaves), 0, s, (const uint16_t *)x,
                       (const uint16_t *)w_router, (const uint16_t *)w_shared_gate, d->T, d->H, d->E, rows, logits);
    return launch_check("moe_route: router_logits_kernel");
}

}  // namespace

namespace moe {

// The logits of a few tokens (T < 32: the one-row-per-workgroup router, no workspace).
moe_status router_logits_small(const moe_route_desc *d, const void *x, const void *w_router, const void *w_shared_gate,
                               float *logits, hipStream_t s) {
    if (router_tiled(d)) {
        set_error("router_logits_small: %d tokens take the tiled router", d->T);
        return MOE_ERR_UNSUPPORTED;
    }
    return enqueue_logits(d, x, w_router, w_shared_gate, logits, nullptr, s);
}

}  // namespace moe

namespace {

double *partial_of(const moe_route_desc *d, void *ws) {
    return (double *)((unsigned char *)ws + align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256));
}

// Checks the routing arguments and enqueues the logits into the workspace.
moe_status route_logits(const moe_route_desc *d, const void *x, const void *w_router, const float *logit_bias,
                        const float *select_bias, const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                        float *shared_gate, void *ws, size_t ws_bytes, hipStream_t s) {
    MOE_REQUIRE(x && w_router && topk_ids && topk_w, "moe_route: NULL x, w_router, topk_ids or topk_w");
    MOE_REQUIRE(!(select_bias && d->score != MOE_SCORE_SIGMOID),
                "moe_route: select_bias is only defined for MOE_SCORE_SIGMOID");
    MOE_REQUIRE((w_shared_gate == nullptr) == (shared_gate == nullptr),
                "moe_route: w_shared_gate and shared_gate must both be given or both NULL");
    const size_t need = moe_route_workspace(d);
    if (!ws || ws_bytes < need) {
        set_error("moe_route: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        return MOE_ERR_WORKSPACE;
    }
    return enqueue_logits(d, x, w_router, w_shared_gate, (float *)ws, partial_of(d, ws), s);
}

}  // namespace

namespace moe {

moe_status check_route_desc(const moe_route_desc *d) { return validate_route(d); }

// The selection half of moe_route_permute (top-k, weights, permutation) from logits already
// computed, for callers inside the library.
moe_status route_select_step(const moe_route_desc *d, const void *ws, const float *logit_bias,
                             const float *select_bias, bool has_sg, int32_t *topk_ids, float *topk_w,
                             float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_to_row,
                             hipStream_t s) {
    if (d->T == 0) return MOE_OK;
    const int rows = d->E + (has_sg ? 1 : 0);
    if (d->T <= 4 && d->T * d->k <= 64)
        return launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, has_sg, topk_ids, topk_w, shared_gate,
                           expert_offsets, sorted_pairs, pair_to_row, s);
    MOE_TRY(launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, has_sg, topk_ids, topk_w, shared_gate,
                        nullptr, nullptr, nullptr, s));
    return moe_permute(d->T, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0,
                       (moe_stream)s);
}

}  // namespace moe

extern "C" moe_status moe_router_logits(const moe_route_desc *d, const void *x, const void *w_router,
                                        const void *w_shared_gate, float *logits, void *ws, size_t ws_bytes,
                                        moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    if (d->T == 0) return MOE_OK;
    MOE_REQUIRE(x && w_router && logits, "moe_router_logits: NULL x, w_router or logits");
    const size_t need = moe_route_workspace(d);
    if (!ws || ws_bytes < need) {
        set_error("moe_router_logits: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        return MOE_ERR_WORKSPACE;
    }
    return enqueue_logits(d, x, w_router, w_shared_gate, logits, partial_of(d, ws), (hipStream_t)stream);
}

extern "C" moe_status moe_route(const moe_route_desc *d, const void *x, const void *w_router,
                                const float *logit_bias, const float *select_bias,
                                const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                float *shared_gate, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    if (d->T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(route_logits(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate, ws,
                         ws_bytes, s));
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    return launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                       topk_w, shared_gate, nullptr, nullptr, nullptr, s);
}

extern "C" moe_status moe_route_permute(const moe_route_desc *d, const void *x, const void *w_router,
                                        const float *logit_bias, const float *select_bias,
                                        const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                        float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                        int32_t *pair_to_row, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    MOE_REQUIRE(expert_offsets != nullptr, "moe_route_permute: NULL expert_offsets");
    MOE_REQUIRE((int64_t)d->T * d->k < INT32_MAX, "moe_route_permute: T*k overflows int32");
    if (d->T > 0) MOE_REQUIRE(sorted_pairs && pair_to_row, "moe_route_permute: NULL sorted_pairs or pair_to_row");
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0) return moe_permute(0, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0,
                                      stream);
    MOE_TRY(route_logits(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate, ws,
                         ws_bytes, s));
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    if (d->T <= 4 && d->T * d->k <= 64)      // one workgroup holds every token: fused permutation
        return launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                           topk_w, shared_gate, expert_offsets, sorted_pairs, pair_to_row, s);
    MOE_TRY(launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                        topk_w, shared_gate, nullptr, nullptr, nullptr, s));
    return moe_permute(d->T, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0, stream);
}

// ------------------------------------------------------------------ no-allocation entry point
// moe_route_permute_noalloc keeps the routing scratch (float32 logits, and for the tiled
// router its float64 split-K partials) in this file-scope device array instead of a
// caller-provided workspace.  Each GPU holds its own copy, at its own address, until the
// process ends; host code uses that address (from hipGetSymbolAddress, once per device),
// never the array's name.  Every call on a GPU shares the array: the kernels overwrite all
// of it that they read, so nothing needs clearing, and calls that overlap on one GPU race.
constexpr size_t kRouteScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kScratchMaxDevices] = {};

// This device's address of `scratch`, looked up on its first use with the device current.
moe_status route_scratch(void **out) {
    int dev = -1;
    MOE_TRY(hip_check(hipGetDevice(&dev), "moe_route_permute_noalloc: hipGetDevice"));
    if (dev < 0 || dev >= kScratchMaxDevices) {
        set_error("moe_route_permute_noalloc: device %d outside [0, %d)", dev, kScratchMaxDevices);
        return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        MOE_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "moe_route_permute_noalloc: hipGetSymbolAddress"));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_route_permute_noalloc(const moe_route_desc *d, const void *x, const void *w_router,
                                                const float *logit_bias, const float *select_bias,
                                                const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                                float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                                int32_t *pair_to_row, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    const size_t need = moe_route_workspace(d);
    if (need > kRouteScratchBytes) {
        set_error("moe_route_permute_noalloc: T = %d, E = %d need %zu bytes of scratch, more than the %zu it holds",
                  d->T, d->E, need, kRouteScratchBytes);
        return MOE_ERR_UNSUPPORTED;
    }
    void *ws = nullptr;
    if (d->T > 0) MOE_TRY(route_scratch(&ws));
    return moe_route_permute(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate,
                             expert_offsets, sorted_pairs, pair_to_row, ws, kRouteScratchBytes, stream);
}

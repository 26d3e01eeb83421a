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

#include "common.h"

namespace moe {
namespace {

constexpr int kRouterTB = 8;      // tokens per wave
constexpr int kRouterUnroll = 4;  // 16-byte loads in flight per lane per pass

// One wave computes the dot products of one weight row (expert e < E, or the shared
// gate row e == E) with up to kRouterTB tokens.  Lanes stride over H in 8-element
// (16-byte) vectors; the float64 partial sums are reduced across the wave in a fixed
// butterfly order.
__global__ __launch_bounds__(64) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ wr,
                                                           const uint16_t *__restrict__ wsg,
                                                           int T, int H, int E, int rows,
                                                           float *__restrict__ logits) {
    const int row = blockIdx.x;
    const uint16_t *w = row < E ? wr + (size_t)row * H : wsg;
    const int t0 = blockIdx.y * kRouterTB;
    const int nt = min(kRouterTB, T - t0);
    const int lane = lane_id();
    double acc[kRouterTB];
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) acc[t] = 0.0;

    const int nvec = H >> 3;
    for (int v0 = lane; v0 < nvec; v0 += kWave * kRouterUnroll) {
        u32x4 wv[kRouterUnroll];
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u) {
            const int v = v0 + u * kWave;
            wv[u] = v < nvec ? __builtin_nontemporal_load((const u32x4 *)(w) + v) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u) {
            const int v = v0 + u * kWave;
            if (v >= nvec) break;
            double wd[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x2 f = bf16x2_to_f32x2(wv[u][q]);
                wd[2 * q] = (double)f.x;
                wd[2 * q + 1] = (double)f.y;
            }
#pragma unroll
            for (int t = 0; t < kRouterTB; ++t) {
                if (t < nt) {
                    const u32x4 xv = ((const u32x4 *)(x + (size_t)(t0 + t) * H))[v];
                    double s = acc[t];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 f = bf16x2_to_f32x2(xv[q]);
                        s = fma(wd[2 * q], (double)f.x, s);
                        s = fma(wd[2 * q + 1], (double)f.y, s);
                    }
                    acc[t] = s;
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) {
        const double s = group_sum_f64(acc[t], kWave);
        if (lane == 0 && t < nt) logits[(size_t)(t0 + t) * rows + row] = (float)s;
    }
}

MOE_DEV double sigmoid_f64(double v) { return 1.0 / (1.0 + exp(-v)); }

// One wave per token: k rounds of a wave-wide argmax over the selection keys (ties to
// the lower expert index), then the weights.  Keys live in LDS; a taken key is set to
// NaN, which never compares greater.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int rows,
                                                   int T, int E, int k, int score, int renorm,
                                                   float scaling, const float *__restrict__ lbias,
                                                   const float *__restrict__ sbias, int has_sg,
                                                   int32_t *__restrict__ ids, float *__restrict__ w,
                                                   float *__restrict__ sg) {
    extern __shared__ double s_key[];
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    double *key = s_key + (size_t)wave_id() * E;
    const int lane = lane_id();
    const float *lt = logits + (size_t)t * rows;

    for (int e = lane; e < E; e += kWave) {
        double l = (double)lt[e] + (lbias ? (double)lbias[e] : 0.0);
        if (score == MOE_SCORE_SIGMOID) l = sigmoid_f64(l) + (sbias ? (double)sbias[e] : 0.0);
        key[e] = l;
    }
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        double bk = -INFINITY;
        int be = INT_MAX;
        for (int e = lane; e < E; e += kWave) {
            const double kv = key[e];
            if (kv > bk || (kv == bk && e < be)) {
                bk = kv;
                be = e;
            }
        }
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const double ok = __shfl_xor(bk, o, kWave);
            const int oe = __shfl_xor(be, o, kWave);
            if (ok > bk || (ok == bk && oe < be)) {
                bk = ok;
                be = oe;
            }
        }
        if (be != INT_MAX && (be & (kWave - 1)) == lane) key[be] = NAN;
        if (lane == j) my_e = be == INT_MAX ? -1 : be;
    }

    const bool mine = lane < k && my_e >= 0;
    double l = 0.0;
    if (mine) l = (double)lt[my_e] + (lbias ? (double)lbias[my_e] : 0.0);
    double wv;
    if (score == MOE_SCORE_SOFTMAX) {
        const double lmax = __shfl(l, 0, kWave);   // first selected = largest logit
        double p = mine ? exp(l - lmax) : 0.0;
        double denom;
        if (renorm) {
            denom = group_sum_f64(p, kWave);
        } else {
            double s = 0.0;
            for (int e = lane; e < E; e += kWave)
                s += exp((double)lt[e] + (lbias ? (double)lbias[e] : 0.0) - lmax);
            denom = group_sum_f64(s, kWave);
        }
        wv = p / denom;
    } else {
        const double s = mine ? sigmoid_f64(l) : 0.0;
        wv = renorm ? s / group_sum_f64(s, kWave) : s;
    }
    wv *= (double)scaling;
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = mine ? (float)wv : NAN;
    }
    if (has_sg && lane == 0) sg[t] = (float)sigmoid_f64((double)lt[E]);
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
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace(const moe_route_desc *d) {
    if (!d || d->T <= 0 || d->E <= 0) return 0;
    return align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256);
}

extern "C" moe_status moe_route(const moe_route_desc *d, const void *x, const void *w_router,
                                const float *logit_bias, const float *select_bias,
                                const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                float *shared_gate, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    if (d->T == 0) return MOE_OK;
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
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    float *logits = (float *)ws;
    hipStream_t s = (hipStream_t)stream;
    dim3 g1(rows, (d->T + kRouterTB - 1) / kRouterTB);
    hipLaunchKernelGGL(router_logits_kernel, g1, dim3(64), 0, s, (const uint16_t *)x,
                       (const uint16_t *)w_router, (const uint16_t *)w_shared_gate, d->T, d->H, d->E,
                       rows, logits);
    MOE_TRY(launch_check("moe_route: router_logits_kernel"));
    const size_t lds = (size_t)4 * d->E * sizeof(double);
    hipLaunchKernelGGL(topk_kernel, dim3((d->T + 3) / 4), dim3(256), lds, s, logits, rows, d->T, d->E,
                       d->k, d->score, d->renormalize, d->routed_scaling, logit_bias, select_bias,
                       w_shared_gate ? 1 : 0, topk_ids, topk_w, shared_gate);
    return launch_check("moe_route: topk_kernel");
}

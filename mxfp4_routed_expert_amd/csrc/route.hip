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
constexpr int kRouterUnroll = 8;  // 16-byte loads in flight per lane per pass

// One wave computes the dot products of one weight row (expert e < E, or the shared gate
// row e == E) with up to kRouterTB tokens.  Lanes stride over H in 8-element (16-byte)
// vectors; loads are issued unconditionally from clamped indices (a load under a branch
// would be waited for at the join) and out-of-range vectors are skipped when consumed.
// The float64 partial sums are reduced across the wave in a fixed butterfly order.
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
    for (int v0 = lane; v0 < nvec + lane; v0 += kWave * kRouterUnroll) {
        u32x4 wv[kRouterUnroll];
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u)
            wv[u] = __builtin_nontemporal_load((const u32x4 *)(w) + min(v0 + u * kWave, nvec - 1));
#pragma unroll
        for (int t = 0; t < kRouterTB; ++t) {
            if (t >= nt) break;                      // uniform across the wave
            const u32x4 *xr = (const u32x4 *)(x + (size_t)(t0 + t) * H);
            u32x4 xv[kRouterUnroll];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) xv[u] = xr[min(v0 + u * kWave, nvec - 1)];
            double s = acc[t];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) {
                if (v0 + u * kWave < nvec) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 fw = bf16x2_to_f32x2(wv[u][q]);
                        const f32x2 fx = bf16x2_to_f32x2(xv[u][q]);
                        s = fma((double)fw.x, (double)fx.x, s);
                        s = fma((double)fw.y, (double)fx.y, s);
                    }
                }
            }
            acc[t] = s;
        }
    }
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) {
        const double s = group_sum_f64(acc[t], kWave);
        if (lane == 0 && t < nt) logits[(size_t)(t0 + t) * rows + row] = (float)s;
    }
}

// Many tokens: a tiled float64 product.  A workgroup owns 128 tokens x 128 rows and one
// of kRouterKS slices of H; bf16 tiles are converted once to float64 into LDS (k-major),
// each thread accumulates an 8 x 8 block of exact products in float64.  The slices' partial
// sums go to the workspace and router_reduce_kernel adds them in a fixed order and rounds
// once to float32 -- the same logits as the one-wave form, up to float64 rounding.
constexpr int kRouterKS = 16;   // K slices
constexpr int kRtTile = 128;
constexpr int kRtKC = 16;       // bf16 values per stage

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ wr,
                                                           const uint16_t *__restrict__ wsg, int T, int H,
                                                           int E, int rows, double *__restrict__ partial) {
    __shared__ __align__(16) double xs[kRtKC][kRtTile];
    __shared__ __align__(16) double wsm[kRtKC][kRtTile];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * kRtTile, r0 = blockIdx.x * kRtTile;
    const int ks = blockIdx.z;
    const int hs = H / kRouterKS;                      // H % (32 * kRouterKS) is checked on the host
    const int h0 = ks * hs, h1 = h0 + hs;
    const int ty = tid >> 4, tx = tid & 15;
    // staging: thread -> (tile row tid/2, 8 values at (tid&1)*8)
    const int lr = tid >> 1, lh = (tid & 1) * 8;
    const int tt = min(t0 + lr, T - 1), rr = min(r0 + lr, rows - 1);
    const bool tok_ok = t0 + lr < T, row_ok = r0 + lr < rows;
    const uint16_t *xrow = x + (size_t)tt * H;
    const uint16_t *wrow = rr < E ? wr + (size_t)rr * H : wsg;
    double acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
    for (int h = h0; h < h1; h += kRtKC) {
        const u32x4 xv = *(const u32x4 *)(xrow + h + lh);
        const u32x4 wv = __builtin_nontemporal_load((const u32x4 *)(wrow + h + lh));
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x2 fx = bf16x2_to_f32x2(xv[q]), fw = bf16x2_to_f32x2(wv[q]);
            xs[lh + 2 * q][lr] = tok_ok ? (double)fx.x : 0.0;
            xs[lh + 2 * q + 1][lr] = tok_ok ? (double)fx.y : 0.0;
            wsm[lh + 2 * q][lr] = row_ok ? (double)fw.x : 0.0;
            wsm[lh + 2 * q + 1][lr] = row_ok ? (double)fw.y : 0.0;
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < kRtKC; ++kk) {
            double a[8], b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = xs[kk][ty * 8 + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = wsm[kk][tx * 8 + j];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = t0 + ty * 8 + i;
        if (t >= T) break;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = r0 + tx * 8 + j;
            if (r < rows) partial[((size_t)ks * T + t) * rows + r] = acc[i][j];
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

MOE_DEV double sigmoid_f64(double v) { return 1.0 / (1.0 + exp(-v)); }

// (key, index) order for selection: larger key first, equal keys -> lower index.
MOE_DEV bool better(double ka, int ia, double kb, int ib) { return ka > kb || (ka == kb && ia < ib); }

template <int CTRL>
MOE_DEV void argmax_dpp_step(double &k, int &i) {
    const int lo = __double2loint(k), hi = __double2hiint(k);
    const int olo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xF, 0xF, false);
    const int ohi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xF, 0xF, false);
    const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
    const double ok = __hiloint2double(ohi, olo);
    if (better(ok, oi, k, i)) {
        k = ok;
        i = oi;
    }
}

// Wave-wide best (key, index): DPP butterfly inside each 16-lane row (quad xor 1, quad
// xor 2, half-row mirror, row mirror), then the four row results through readlane.
MOE_DEV void wave_argmax(double &k, int &i) {
    argmax_dpp_step<0xB1>(k, i);    // quad_perm(1,0,3,2)
    argmax_dpp_step<0x4E>(k, i);    // quad_perm(2,3,0,1)
    argmax_dpp_step<0x141>(k, i);   // row_half_mirror
    argmax_dpp_step<0x140>(k, i);   // row_mirror
    double bk = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(k), 0),
                                 __builtin_amdgcn_readlane(__double2loint(k), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const double rk = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(k), 16 * r),
                                           __builtin_amdgcn_readlane(__double2loint(k), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (better(rk, ri, bk, bi)) {
            bk = rk;
            bi = ri;
        }
    }
    k = bk;
    i = bi;
}

// One wave per token.  Lane l holds the selection keys of experts l, l+64, ... in
// registers and tracks its own best untaken key; each of the k rounds takes the wave-wide
// best (ties to the lower expert index) and only the winning lane rescans its keys.
// A NaN key is never selected (ids -1 are emitted if fewer than k keys compare).
template <int NK>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int rows,
                                                   int T, int E, int k, int score, int renorm,
                                                   float scaling, const float *__restrict__ lbias,
                                                   const float *__restrict__ sbias, int has_sg,
                                                   int32_t *__restrict__ ids, float *__restrict__ w,
                                                   float *__restrict__ sg) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    const int lane = lane_id();
    const float *lt = logits + (size_t)t * rows;

    double key[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        double l = (double)lt[e] + (lbias ? (double)lbias[e] : 0.0);
        if (score == MOE_SCORE_SIGMOID) l = sigmoid_f64(l) + (sbias ? (double)sbias[e] : 0.0);
        key[i] = lane + 64 * i < E ? l : NAN;
    }
    uint32_t taken = 0;
    auto local_best = [&](double &bk, int &bi) {
        bk = -INFINITY;
        bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int e = lane + 64 * i;
            if (!((taken >> i) & 1u) && better(key[i], e, bk, bi)) {
                bk = key[i];
                bi = e;
            }
        }
    };
    double lk;
    int li;
    local_best(lk, li);
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        double wk = lk;
        int wi = li;
        wave_argmax(wk, wi);
        if (lane == j) my_e = wi == INT_MAX ? -1 : wi;
        if (wi != INT_MAX && (wi & 63) == lane) {     // the winner drops its key
            taken |= 1u << (wi >> 6);
            local_best(lk, li);
        }
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
        const double sv = mine ? sigmoid_f64(l) : 0.0;
        wv = renorm ? sv / group_sum_f64(sv, kWave) : sv;
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
    size_t b = align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256);
    if (d->H % 32 == 0 && router_tiled(d)) b += (size_t)kRouterKS * d->T * (d->E + 1) * sizeof(double);
    return b;
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
    if (router_tiled(d)) {
        double *partial = (double *)((unsigned char *)ws + align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256));
        dim3 gt((rows + kRtTile - 1) / kRtTile, (d->T + kRtTile - 1) / kRtTile, kRouterKS);
        hipLaunchKernelGGL(router_tiled_kernel, gt, dim3(256), 0, s, (const uint16_t *)x, (const uint16_t *)w_router,
                           (const uint16_t *)w_shared_gate, d->T, d->H, d->E, rows, partial);
        MOE_TRY(launch_check("moe_route: router_tiled_kernel"));
        const int n = d->T * rows;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, partial, n, logits);
        MOE_TRY(launch_check("moe_route: router_reduce_kernel"));
    } else {
        dim3 g1(rows, (d->T + kRouterTB - 1) / kRouterTB);
        hipLaunchKernelGGL(router_logits_kernel, g1, dim3(64), 0, s, (const uint16_t *)x,
                           (const uint16_t *)w_router, (const uint16_t *)w_shared_gate, d->T, d->H, d->E,
                           rows, logits);
        MOE_TRY(launch_check("moe_route: router_logits_kernel"));
    }
    auto topk = d->E <= 256 ? topk_kernel<4> : d->E <= 512 ? topk_kernel<8> : d->E <= 1024 ? topk_kernel<16>
                                                                                           : topk_kernel<32>;
    const int tb = d->T < 4 ? 64 * d->T : 256;
    hipLaunchKernelGGL(topk, dim3((d->T + 3) / 4), dim3(tb), 0, s, logits, rows, d->T, d->E, d->k, d->score,
                       d->renormalize, d->routed_scaling, logit_bias, select_bias, w_shared_gate ? 1 : 0,
                       topk_ids, topk_w, shared_gate);
    return launch_check("moe_route: topk_kernel");
}

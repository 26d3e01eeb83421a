// One router weight row against a few tokens: the per-quarter partial sums of the decode
// router (router_logits_kernel in route.hip) and of the single-launch decode step
// (decode_step_kernel in gemv.hip), which therefore produce the same logits bit for bit.
//
// The logit of (t, e) is the float32 rounding of the exact dot product of two bf16 vectors
// (rabbit README, architecture table: softmax and noaux_tc sigmoid routing over these
// logits): bf16 x bf16 products are exact in float64, the sum is accumulated in float64 and
// rounded once.
#pragma once

#include "common.h"

namespace moe {

constexpr int kRouterTB = 8;      // tokens per wave
constexpr int kRouterUnroll = 4;  // 16-byte loads in flight per lane per pass
constexpr int kRouterWaves = 4;   // waves per row, one quarter of H each

// Wave `quarter` of a row's four covers that quarter of H (H % 32 == 0, so quarters are
// whole 16-byte vectors); lanes stride over it in 8-element vectors, loads issued
// unconditionally from clamped indices (a load under a branch would be waited for at the
// join) and out-of-range vectors skipped when consumed.  Returns, in every lane, the
// wave's float64 partial sums of tokens t0 .. t0 + nt - 1, reduced over the wave in a fixed
// butterfly order.  The row's logit is the sum of the four quarters in quarter order.
MOE_DEV void router_quarter(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int t0, int nt, int H,
                            int quarter, double (&out)[kRouterTB]) {
    const int lane = lane_id();
    double acc[kRouterTB];
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) acc[t] = 0.0;
    const int nvec = H >> 3;
    const int q0 = quarter * (nvec / kRouterWaves), q1 = q0 + nvec / kRouterWaves;
    for (int v0 = q0 + lane; v0 < q1 + lane; v0 += kWave * kRouterUnroll) {
        u32x4 wv[kRouterUnroll];
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u)
            wv[u] = __builtin_nontemporal_load((const u32x4 *)(w) + min(v0 + u * kWave, q1 - 1));
#pragma unroll
        for (int t = 0; t < kRouterTB; ++t) {
            if (t >= nt) break;                      // uniform across the wave
            const u32x4 *xr = (const u32x4 *)(x + (size_t)(t0 + t) * H);
            u32x4 xv[kRouterUnroll];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) xv[u] = xr[min(v0 + u * kWave, q1 - 1)];
            double s = acc[t];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) {
                if (v0 + u * kWave < q1) {
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
        if (t >= nt) break;                          // (each reduction is a chain of shuffles)
        out[t] = group_sum_f64(acc[t], kWave);
    }
}

// The row's logit of token t from its quarters' partial sums part[quarter][t].
MOE_DEV float router_finish(const double (*part)[kRouterTB], int t) {
    double s = 0.0;
#pragma unroll
    for (int w4 = 0; w4 < kRouterWaves; ++w4) s += part[w4][t];
    return (float)s;
}

}  // namespace moe

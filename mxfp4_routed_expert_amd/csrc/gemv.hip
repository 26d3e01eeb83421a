// Decode-path dequant-GEMV for the expert FFN (and the bf16 LatentMoE projections).
//
// The pages' decode is bound by streaming expert bytes: "59% waiting for expert bytes,
// 31% multiplying them" (rabbit README, design section) and Rulith's decode "reads the
// weights at the memory's speed" (Rulith Inference README, engine section).  With all
// experts resident in HBM the whole product is one HBM stream, so the kernel is built
// around the weight bytes:
//   * every lane loads 16 bytes per step -- exactly one MXFP4 block of 32 weights (or
//     16 FP8 weights, or 8 bf16 weights) -- and the G lanes that share a matrix row read
//     consecutive 16-byte units, so each wave-wide load is a set of contiguous
//     G*16-byte segments; weights are read with non-temporal loads (used once);
//   * codes are converted in registers by the gfx950 scaled-conversion instructions
//     (E2M1/E4M3 -> bf16 or f32, unscaled), dotted with activations staged in LDS, and
//     the block's E8M0 (or FP8 tile) scale is applied once per block to the partial sum;
//   * for the gate/up pair, lanes 0-31 of a wave read a gate row and lanes 32-63 the up
//     row with the same index, so SwiGLU is applied in registers after the reduction
//     and h is written once;
//   * a workgroup owns one expert and a range of rows; the expert is found from
//     expert_offsets on the device (the slot-th expert that has rows), so no host
//     synchronisation is needed and empty experts cost nothing.
#include "gemv.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvUnroll = 8;

template <int FMT>
MOE_DEV int units_per_row(int K) {
    return FMT == kFmtMXFP4 ? K / 32 : (FMT == kFmtFP8 ? K / 16 : K / 8);
}

// Partial dot product of one 16-byte weight unit with activation row `a` (in LDS),
// before the unit's scale.  Unit b covers elements [b*EPU, (b+1)*EPU).
template <int FMT, bool ACT_F32>
MOE_DEV float unit_dot(const u32x4 wv, const void *a_unit) {
    float s = 0.0f;
    if constexpr (!ACT_F32) {
        const u32x4 *a4 = (const u32x4 *)a_unit;
        if constexpr (FMT == kFmtMXFP4) {
            // 32 codes: dword d holds elements 8d..8d+7, byte q -> elements 8d+2q, 8d+2q+1
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x4 av = a4[d];
                s = dot2_bf16(fp4x2_to_bf16x2<0>(wv[d]), as_bf16x2(av[0]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<1>(wv[d]), as_bf16x2(av[1]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<2>(wv[d]), as_bf16x2(av[2]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<3>(wv[d]), as_bf16x2(av[3]), s);
            }
        } else if constexpr (FMT == kFmtFP8) {
            // 16 codes: dword d holds elements 4d..4d+3
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 av = a4[h];
                s = dot2_bf16(fp8x2_to_bf16x2<false>(wv[2 * h]), as_bf16x2(av[0]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<true>(wv[2 * h]), as_bf16x2(av[1]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<false>(wv[2 * h + 1]), as_bf16x2(av[2]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<true>(wv[2 * h + 1]), as_bf16x2(av[3]), s);
            }
        } else {
            const u32x4 av = a4[0];
#pragma unroll
            for (int d = 0; d < 4; ++d) s = dot2_bf16(as_bf16x2(wv[d]), as_bf16x2(av[d]), s);
        }
    } else {
        const f32x4 *a4 = (const f32x4 *)a_unit;
        if constexpr (FMT == kFmtMXFP4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x4 lo = a4[2 * d], hi = a4[2 * d + 1];
                f32x2 w0 = fp4x2_to_f32x2<0>(wv[d]), w1 = fp4x2_to_f32x2<1>(wv[d]);
                f32x2 w2 = fp4x2_to_f32x2<2>(wv[d]), w3 = fp4x2_to_f32x2<3>(wv[d]);
                s = fmaf(w0.x, lo[0], s); s = fmaf(w0.y, lo[1], s);
                s = fmaf(w1.x, lo[2], s); s = fmaf(w1.y, lo[3], s);
                s = fmaf(w2.x, hi[0], s); s = fmaf(w2.y, hi[1], s);
                s = fmaf(w3.x, hi[2], s); s = fmaf(w3.y, hi[3], s);
            }
        } else if constexpr (FMT == kFmtFP8) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x4 av = a4[d];
                f32x2 w0 = fp8x2_to_f32x2<false>(wv[d]), w1 = fp8x2_to_f32x2<true>(wv[d]);
                s = fmaf(w0.x, av[0], s); s = fmaf(w0.y, av[1], s);
                s = fmaf(w1.x, av[2], s); s = fmaf(w1.y, av[3], s);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 av = a4[h];
                f32x2 w0 = bf16x2_to_f32x2(wv[2 * h]), w1 = bf16x2_to_f32x2(wv[2 * h + 1]);
                s = fmaf(w0.x, av[0], s); s = fmaf(w0.y, av[1], s);
                s = fmaf(w1.x, av[2], s); s = fmaf(w1.y, av[3], s);
            }
        }
    }
    return s;
}

// Activation staging: rows of the token chunk are copied to LDS unchanged (bf16, f32) or,
// for MX-quantised activations, decoded block by block to bf16 (E2M1 * 2^X is exact in
// bf16).  Rows whose index is out of range are staged as zeros.
template <int ACT>
MOE_DEV void stage_activations(const GemvParams &p, unsigned char *smem, int row0, int c0, int mc) {
    constexpr int ASZ = ACT == kActF32 ? 4 : 2;
    const int K = p.K;
    if constexpr (ACT == kActMX) {
        const int nb = K / 32;
        for (int i = threadIdx.x; i < mc * nb; i += kGemvThreads) {
            const int m = i / nb, blk = i - m * nb;
            const int r = row0 + c0 + m;
            int arow = p.gather ? p.sorted_pairs[r] : r;
            if (p.gather) arow = arow >= 0 ? arow / p.k : -1;
            u32x4 *dst = (u32x4 *)(smem + ((size_t)m * K + (size_t)blk * 32) * 2);
            if (arow >= 0 && arow < p.n_act_rows) {
                const u32x4 cv = ((const u32x4 *)((const uint8_t *)p.act + (size_t)arow * (K / 2)))[blk];
                const float sc = e8m0_to_f32(p.act_s[(size_t)arow * nb + blk]);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 0);
                    const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 1);
                    const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 2);
                    const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 3);
                    dst[d] = u32x4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                   __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
                }
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d) dst[d] = u32x4{0, 0, 0, 0};
            }
        }
    } else {
        const int act_vec = K * ASZ / 16;      // 16-byte vectors per activation row
        for (int i = threadIdx.x; i < mc * act_vec; i += kGemvThreads) {
            const int m = i / act_vec, v = i - m * act_vec;
            const int r = row0 + c0 + m;
            int arow = p.gather ? p.sorted_pairs[r] : r;
            if (p.gather) arow = arow >= 0 ? arow / p.k : -1;
            u32x4 val = {0, 0, 0, 0};
            if (arow >= 0 && arow < p.n_act_rows)
                val = ((const u32x4 *)((const unsigned char *)p.act + (size_t)arow * K * ASZ))[v];
            ((u32x4 *)smem)[i] = val;
        }
    }
}

template <int FMT, int ACT, int MAXM, bool PAIR, bool ROUTED>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const GemvParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_scan[kGemvThreads / 64 + 1];
    constexpr bool ACT_F32 = ACT == kActF32;
    constexpr int ASZ = ACT_F32 ? 4 : 2;
    constexpr int EPU = FMT == kFmtMXFP4 ? 32 : (FMT == kFmtFP8 ? 16 : 8);   // elements per unit

    int e = 0, row0 = 0, M = p.T;
    if constexpr (ROUTED) {
        e = nth_nonempty_expert(p.offsets, p.E, blockIdx.y, s_scan);
        if (e < 0) return;
        row0 = p.offsets[e];
        M = p.offsets[e + 1] - row0;
        if (row0 < 0 || M <= 0 || row0 + M > p.R) return;
    }
    const int K = p.K;
    const int units = units_per_row<FMT>(K);
    const int lane = lane_id(), wave = wave_id();
    const int G = p.G;
    const int rows_per_pass = PAIR ? 32 / G : 64 / G;
    const int grp = PAIR ? (lane & 31) / G : lane / G;
    const int j = lane & (G - 1);
    const int mat = PAIR ? (lane >> 5) : 0;
    const uint8_t *W = p.w[mat];
    const int n_begin = blockIdx.x * p.rows_per_wg;
    const int n_end = min(p.N, n_begin + p.rows_per_wg);
    if (n_begin >= n_end) return;
    const int passes = (n_end - n_begin + rows_per_pass - 1) / rows_per_pass;
    const size_t row_bytes = (size_t)units * 16;

    for (int c0 = 0; c0 < M; c0 += p.chunk) {
        const int mc = min(p.chunk, M - c0);
        __syncthreads();
        stage_activations<ACT>(p, smem, row0, c0, mc);
        __syncthreads();

        for (int pass = wave; pass < passes; pass += kGemvThreads / 64) {
            const int n = n_begin + pass * rows_per_pass + grp;
            const bool row_ok = n < n_end;
            const size_t ridx = (size_t)e * p.N + (row_ok ? n : 0);
            const uint8_t *wrow = W + ridx * row_bytes;
            float acc[MAXM];
#pragma unroll
            for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;

            for (int i0 = 0; i0 < p.nl; i0 += kGemvUnroll) {
                u32x4 wv[kGemvUnroll];
                float sc[kGemvUnroll];
#pragma unroll
                for (int u = 0; u < kGemvUnroll; ++u) {
                    const int b = j + (i0 + u) * G;
                    const bool ok = row_ok && (i0 + u) < p.nl && b < units;
                    wv[u] = u32x4{0, 0, 0, 0};
                    sc[u] = 0.0f;
                    if (ok) {
                        wv[u] = __builtin_nontemporal_load((const u32x4 *)(wrow + (size_t)b * 16));
                        if constexpr (FMT == kFmtMXFP4) {
                            sc[u] = e8m0_to_f32(((const uint8_t *)p.s[mat])[ridx * units + b]);
                        } else if constexpr (FMT == kFmtFP8) {
                            const size_t srow = (size_t)e * (p.N / 128) + n / 128;
                            sc[u] = ((const float *)p.s[mat])[srow * (K / 128) + (b * 16) / 128];
                        } else {
                            sc[u] = 1.0f;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kGemvUnroll; ++u) {
                    const int b = j + (i0 + u) * G;
                    const bool ok = row_ok && (i0 + u) < p.nl && b < units;
                    if (ok) {
#pragma unroll
                        for (int m = 0; m < MAXM; ++m) {
                            if (m < mc) {
                                const void *a = smem + ((size_t)m * K + (size_t)b * EPU) * ASZ;
                                acc[m] = fmaf(unit_dot<FMT, ACT_F32>(wv[u], a), sc[u], acc[m]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MAXM; ++m) acc[m] = group_sum(acc[m], G);
            if constexpr (PAIR) {
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    const float up = __shfl_xor(acc[m], 32, kWave);
                    acc[m] = silu(acc[m]) * up;
                }
            }
            if (row_ok && j == 0 && mat == 0) {
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    if (m < mc) {
                        const size_t o = (size_t)(row0 + c0 + m) * p.N + n;
                        float v = acc[m];
                        if (p.residual) v += p.residual[o];
                        p.out[o] = v;
                    }
                }
            }
        }
    }
}

// Lanes per row and units per lane for a row of `units` 16-byte units: the widest group
// that still gives each lane >= 6 units with at most 1/8 of the lanes' slots idle.
static void pick_layout(int units, bool pair, int *G, int *nl) {
    const int cands[] = {64, 32, 16, 8, 4};
    for (int g : cands) {
        if (pair && g > 32) continue;
        const int n = (units + g - 1) / g;
        if (n >= 6 && (n * g - units) * 8 <= n * g) {
            *G = g;
            *nl = n;
            return;
        }
    }
    *G = 4;
    *nl = (units + 3) / 4;
}

using GemvFn = void (*)(const GemvParams);

template <int FMT, int ACT, bool PAIR>
static GemvFn pick_kernel_m(int maxm, bool routed) {
    if (routed) {
        switch (maxm) {
            case 1: return gemv_kernel<FMT, ACT, 1, PAIR, true>;
            case 2: return gemv_kernel<FMT, ACT, 2, PAIR, true>;
            case 4: return gemv_kernel<FMT, ACT, 4, PAIR, true>;
            default: return gemv_kernel<FMT, ACT, 8, PAIR, true>;
        }
    }
    switch (maxm) {
        case 1: return gemv_kernel<FMT, ACT, 1, PAIR, false>;
        case 2: return gemv_kernel<FMT, ACT, 2, PAIR, false>;
        case 4: return gemv_kernel<FMT, ACT, 4, PAIR, false>;
        default: return gemv_kernel<FMT, ACT, 8, PAIR, false>;
    }
}

template <int FMT, bool PAIR>
static GemvFn pick_kernel_a(int act, int maxm, bool routed) {
    if (act == kActF32) return pick_kernel_m<FMT, kActF32, PAIR>(maxm, routed);
    if (act == kActMX && FMT == kFmtMXFP4) return pick_kernel_m<kFmtMXFP4, kActMX, PAIR>(maxm, routed);
    return pick_kernel_m<FMT, kActBF16, PAIR>(maxm, routed);
}

static GemvFn pick_kernel(int fmt, int act, bool pair, int maxm, bool routed) {
    if (fmt == kFmtMXFP4)
        return pair ? pick_kernel_a<kFmtMXFP4, true>(act, maxm, routed) : pick_kernel_a<kFmtMXFP4, false>(act, maxm, routed);
    if (fmt == kFmtFP8)
        return pair ? pick_kernel_a<kFmtFP8, true>(act, maxm, routed) : pick_kernel_a<kFmtFP8, false>(act, maxm, routed);
    return pick_kernel_a<kFmtBF16, false>(act, maxm, false);
}

constexpr size_t kGemvLdsBudget = 64 * 1024;

moe_status gemv_launch(int fmt, int act, bool pair, GemvParams p, int slots, int max_rows_per_expert,
                       hipStream_t stream, const char *what) {
    const bool act_f32 = act == kActF32;
    const int units = fmt == kFmtMXFP4 ? p.K / 32 : (fmt == kFmtFP8 ? p.K / 16 : p.K / 8);
    pick_layout(units, pair, &p.G, &p.nl);
    int maxm = 1;
    while (maxm < max_rows_per_expert && maxm < 8) maxm *= 2;
    const size_t row_lds = (size_t)p.K * (act_f32 ? 4 : 2);
    int chunk = (int)(kGemvLdsBudget / row_lds);
    if (chunk < 1) {
        set_error("%s: an activation row of %zu bytes does not fit the LDS budget", what, row_lds);
        return MOE_ERR_UNSUPPORTED;
    }
    p.chunk = chunk < maxm ? chunk : maxm;
    const int rows_per_pass = pair ? 32 / p.G : 64 / p.G;
    // aim for ~2048 workgroups over the whole launch, at least one pass per wave
    long long rows_total = (long long)p.N * slots;
    int rpw = (int)(rows_total / 2048);
    const int min_rpw = rows_per_pass * (kGemvThreads / 64);
    if (rpw < min_rpw) rpw = min_rpw;
    rpw = (rpw + rows_per_pass - 1) / rows_per_pass * rows_per_pass;
    p.rows_per_wg = rpw;
    dim3 grid((p.N + rpw - 1) / rpw, slots);
    const size_t lds = (size_t)p.chunk * row_lds;
    GemvFn fn = pick_kernel(fmt, act, pair, maxm, p.offsets != nullptr);
    hipLaunchKernelGGL(fn, grid, dim3(kGemvThreads), lds, stream, p);
    return launch_check(what);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_dense_bf16(int32_t T, int32_t n, int32_t kdim, const void *x, int32_t x_dtype,
                                     const void *w, const float *residual, float *y, moe_stream stream) {
    clear_error();
    MOE_REQUIRE(T >= 0 && n > 0 && kdim > 0 && kdim % 8 == 0,
                "moe_dense_bf16: need T >= 0, n > 0, kdim > 0 and a multiple of 8 (T=%d n=%d kdim=%d)", T, n,
                kdim);
    MOE_REQUIRE(x_dtype == MOE_DT_BF16 || x_dtype == MOE_DT_F32, "moe_dense_bf16: unknown x_dtype %d", x_dtype);
    MOE_REQUIRE((int64_t)T * n < INT32_MAX && (int64_t)n * kdim < INT32_MAX && (int64_t)T * kdim < INT32_MAX,
                "moe_dense_bf16: sizes overflow int32");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(x && w && y, "moe_dense_bf16: NULL x, w or y");
    GemvParams p = {};
    p.w[0] = (const uint8_t *)w;
    p.N = n;
    p.K = kdim;
    p.E = 1;
    p.act = x;
    p.gather = 0;
    p.n_act_rows = T;
    p.T = T;
    p.R = T;
    p.out = y;
    p.residual = residual;
    return gemv_launch(kFmtBF16, x_dtype == MOE_DT_F32 ? kActF32 : kActBF16, false, p, 1, T,
                       (hipStream_t)stream, "moe_dense_bf16");
}

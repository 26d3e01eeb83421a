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

// Tuning constants (compile-time; -D overrides build variants for sweeps).
#ifndef MOE_GEMV_UNROLL
#define MOE_GEMV_UNROLL 4        // 16-byte weight loads issued per lane per batch
#endif
#ifndef MOE_GEMV_DEPTH
#define MOE_GEMV_DEPTH 2         // batches in flight per wave (deeper measured slower: more
                                 // registers, and no faster streaming at this occupancy)
#endif
#ifndef MOE_GEMV_TARGET_WG
#define MOE_GEMV_TARGET_WG 1024  // workgroups a launch aims for
#endif
#ifndef MOE_GEMV_NT
#define MOE_GEMV_NT 1            // non-temporal weight loads
#endif
#ifndef MOE_GEMV_WAVES_PER_EU
#define MOE_GEMV_WAVES_PER_EU 0  // occupancy hint (0: compiler's choice)
#endif
constexpr int kGemvThreads = 256;
constexpr int kGemvUnroll = MOE_GEMV_UNROLL;
constexpr int kGemvDepth = MOE_GEMV_DEPTH;
#if MOE_GEMV_WAVES_PER_EU > 0
#define MOE_GEMV_ATTR __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(MOE_GEMV_WAVES_PER_EU)))
#else
#define MOE_GEMV_ATTR __launch_bounds__(kGemvThreads)
#endif

template <int FMT>
MOE_DEV int units_per_row(int K) {
    return FMT == kFmtMXFP4 ? K / 32 : (FMT == kFmtFP8 ? K / 16 : K / 8);
}

// Activations in LDS: the elements of weight unit b occupy P = bytes/16 consecutive 16-byte
// slots, with slot s stored at position s ^ swz(b).  Lanes of a row group read consecutive
// units; without the swizzle the lanes a bank period apart would read the same banks.
template <int FMT, bool ACT_F32>
constexpr int act_slots() {
    return ((FMT == 0 ? 32 : (FMT == 1 ? 16 : 8)) * (ACT_F32 ? 4 : 2)) / 16;
}
template <int FMT, bool ACT_F32>
MOE_DEV int act_swizzle(int b) {
    constexpr int P = act_slots<FMT, ACT_F32>();
    constexpr int per_period = 256 / (16 * P);   // units per 256-byte bank period
    if constexpr (P == 1) return 0;
    else return (b / per_period) & (P - 1);
}

// Partial dot product of one 16-byte weight unit with activation row `a` (in LDS, slots
// swizzled with key `z`), before the unit's scale.  Unit b covers elements [b*EPU, (b+1)*EPU).
template <int FMT, bool ACT_F32>
MOE_DEV float unit_dot(const u32x4 wv, const void *a_unit, int z) {
    float s = 0.0f;
    if constexpr (!ACT_F32) {
        const u32x4 *a4s = (const u32x4 *)a_unit;
        auto a4 = [&](int i) { return a4s[i ^ z]; };
        if constexpr (FMT == kFmtMXFP4) {
            // 32 codes: dword d holds elements 8d..8d+7, byte q -> elements 8d+2q, 8d+2q+1
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x4 av = a4(d);
                s = dot2_bf16(fp4x2_to_bf16x2<0>(wv[d]), as_bf16x2(av[0]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<1>(wv[d]), as_bf16x2(av[1]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<2>(wv[d]), as_bf16x2(av[2]), s);
                s = dot2_bf16(fp4x2_to_bf16x2<3>(wv[d]), as_bf16x2(av[3]), s);
            }
        } else if constexpr (FMT == kFmtFP8) {
            // 16 codes: dword d holds elements 4d..4d+3
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 av = a4(h);
                s = dot2_bf16(fp8x2_to_bf16x2<false>(wv[2 * h]), as_bf16x2(av[0]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<true>(wv[2 * h]), as_bf16x2(av[1]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<false>(wv[2 * h + 1]), as_bf16x2(av[2]), s);
                s = dot2_bf16(fp8x2_to_bf16x2<true>(wv[2 * h + 1]), as_bf16x2(av[3]), s);
            }
        } else {
            const u32x4 av = a4(0);
#pragma unroll
            for (int d = 0; d < 4; ++d) s = dot2_bf16(as_bf16x2(wv[d]), as_bf16x2(av[d]), s);
        }
    } else {
        const f32x4 *a4s = (const f32x4 *)a_unit;
        auto a4 = [&](int i) { return a4s[i ^ z]; };
        if constexpr (FMT == kFmtMXFP4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x4 lo = a4(2 * d), hi = a4(2 * d + 1);
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
                const f32x4 av = a4(d);
                f32x2 w0 = fp8x2_to_f32x2<false>(wv[d]), w1 = fp8x2_to_f32x2<true>(wv[d]);
                s = fmaf(w0.x, av[0], s); s = fmaf(w0.y, av[1], s);
                s = fmaf(w1.x, av[2], s); s = fmaf(w1.y, av[3], s);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 av = a4(h);
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
template <int FMT, int ACT>
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
            const int z = act_swizzle<kFmtMXFP4, false>(blk);
            if (arow >= 0 && arow < p.n_act_rows) {
                const u32x4 cv = ((const u32x4 *)((const uint8_t *)p.act + (size_t)arow * (K / 2)))[blk];
                const float sc = e8m0_to_f32(p.act_s[(size_t)arow * nb + blk]);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 0);
                    const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 1);
                    const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 2);
                    const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[d], sc, 3);
                    dst[d ^ z] = u32x4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
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
            constexpr int P = act_slots<FMT, ACT == kActF32>();
            const int b = v / P, sl = v - b * P;
            ((u32x4 *)smem)[(size_t)m * act_vec + b * P + (sl ^ act_swizzle<FMT, ACT == kActF32>(b))] = val;
        }
    }
}

// Geometry of one wave's share of a workgroup's rows.  A wave walks its passes (one pass =
// the rows_per_pass rows its lane groups own at once) as a stream of batches of
// kGemvUnroll 16-byte units per lane; batch q covers pass q / nb, units [i0, i0 + U).
struct WaveStream {
    int n_first;     // row of this lane group in the wave's first pass
    int row_step;    // rows between consecutive passes of this wave
    int nb;          // batches per pass
    int nbatch;      // batches of this wave
    int n_end;
};

// wbase / sbase: this lane's matrix (gate or up for the pair), chosen once per kernel with a
// select -- indexing the parameter arrays by a lane-dependent value would load the pointer
// from memory on every use.  Every load is issued unconditionally from a clamped, valid
// address: a load under a branch would make the compiler wait for it (and, loads retiring
// in order, for every load before it) where the branch joins.  Slots past the row or the
// row range are skipped when the batch is consumed.  Scale bytes stay raw until then.
template <int FMT>
MOE_DEV void load_batch(const GemvParams &p, const WaveStream &ws, int q, int e, const uint8_t *wbase,
                        const void *sbase, int j, int units, u32x4 (&w)[kGemvUnroll], uint32_t (&sc)[kGemvUnroll]) {
    const int pi = q / ws.nb;
    const int i0 = (q - pi * ws.nb) * kGemvUnroll;
    const int n = min(ws.n_first + pi * ws.row_step, ws.n_end - 1);
    const size_t ridx = (size_t)e * p.N + n;
    const uint8_t *wrow = wbase + ridx * (size_t)units * 16;
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
        const int b = min(j + (i0 + u) * p.G, units - 1);
#if MOE_GEMV_NT
        w[u] = __builtin_nontemporal_load((const u32x4 *)(wrow + (size_t)b * 16));
#else
        w[u] = *(const u32x4 *)(wrow + (size_t)b * 16);
#endif
        if constexpr (FMT == kFmtMXFP4) {
            sc[u] = ((const uint8_t *)sbase)[ridx * units + b];
        } else if constexpr (FMT == kFmtFP8) {
            const size_t srow = (size_t)e * (p.N / 128) + n / 128;
            sc[u] = __float_as_uint(((const float *)sbase)[srow * (p.K / 128) + (b * 16) / 128]);
        } else {
            sc[u] = 0;
        }
    }
}

MOE_DEV float unit_scale_value(int fmt, uint32_t raw) {
    return fmt == kFmtMXFP4 ? e8m0_to_f32(raw) : (fmt == kFmtFP8 ? __uint_as_float(raw) : 1.0f);
}

// Accumulate batch q into acc; after the last batch of a pass, reduce over the lane group,
// apply SwiGLU for the gate/up pair, write the rows and clear acc.  Called by the whole
// wave with the same q (the reductions are wave-wide shuffles).
template <int FMT, int ACT, int MAXM, bool PAIR>
MOE_DEV void compute_batch(const GemvParams &p, const WaveStream &ws, int q, int mat, int j, int units,
                           const unsigned char *smem, int out_row0, int mc, const u32x4 (&w)[kGemvUnroll],
                           const uint32_t (&sc)[kGemvUnroll], float (&acc)[MAXM]) {
    constexpr bool ACT_F32 = ACT == kActF32;
    constexpr int ASZ = ACT_F32 ? 4 : 2;
    constexpr int EPU = FMT == kFmtMXFP4 ? 32 : (FMT == kFmtFP8 ? 16 : 8);
    const int pi = q / ws.nb;
    const int ib = q - pi * ws.nb;
    const int i0 = ib * kGemvUnroll;
    const int n = ws.n_first + pi * ws.row_step;
    const bool row_ok = n < ws.n_end;
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
        const int b = j + (i0 + u) * p.G;
        if (row_ok && (i0 + u) < p.nl && b < units) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < mc) {
                    const void *a = smem + ((size_t)m * p.K + (size_t)b * EPU) * ASZ;
                    acc[m] = fmaf(unit_dot<FMT, ACT_F32>(w[u], a, act_swizzle<FMT, ACT_F32>(b)),
                                  unit_scale_value(FMT, sc[u]), acc[m]);
                }
            }
        }
    }
    if (ib != ws.nb - 1) return;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = group_sum(acc[m], p.G);
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
                const size_t o = (size_t)(out_row0 + m) * p.N + n;
                float v = acc[m];
                if (p.residual) v += p.residual[o];
                p.out[o] = v;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
}

template <int FMT, int ACT, int MAXM, bool PAIR, bool ROUTED>
__global__ MOE_GEMV_ATTR void gemv_kernel(const GemvParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = kGemvThreads / 64;

    int e = 0, row0 = 0, M = p.T;
    if constexpr (ROUTED) {
        e = wave_nth_nonempty(p.offsets, p.E, blockIdx.y);
        if (e < 0) return;
        row0 = p.offsets[e];
        M = p.offsets[e + 1] - row0;
        if (row0 < 0 || M <= 0 || row0 + M > p.R) return;
    }
    const int units = units_per_row<FMT>(p.K);
    const int lane = lane_id(), wave = wave_id();
    const int G = p.G;
    const int rows_per_pass = PAIR ? 32 / G : 64 / G;
    const int grp = PAIR ? (lane & 31) / G : lane / G;
    const int j = lane & (G - 1);
    const int mat = PAIR ? (lane >> 5) : 0;
    const uint8_t *wbase = PAIR && mat ? p.w[1] : p.w[0];
    const void *sbase = PAIR && mat ? p.s[1] : p.s[0];
    const int n_begin = blockIdx.x * p.rows_per_wg;
    const int n_end = min(p.N, n_begin + p.rows_per_wg);
    if (n_begin >= n_end) return;
    const int passes = (n_end - n_begin + rows_per_pass - 1) / rows_per_pass;
    WaveStream ws;
    ws.n_first = n_begin + wave * rows_per_pass + grp;
    ws.row_step = NW * rows_per_pass;
    ws.nb = (p.nl + kGemvUnroll - 1) / kGemvUnroll;
    ws.nbatch = (wave < passes ? (passes - 1 - wave) / NW + 1 : 0) * ws.nb;
    ws.n_end = n_end;

    // batches rotate through kGemvDepth register buffers: while batch q is consumed, the
    // next kGemvDepth-1 are in flight
    u32x4 wbuf[kGemvDepth][kGemvUnroll];
    uint32_t sbuf[kGemvDepth][kGemvUnroll];
    float acc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;

    for (int c0 = 0; c0 < M; c0 += p.chunk) {
        const int mc = min(p.chunk, M - c0);
        // the first weight batches are in flight while the activations are staged
#pragma unroll
        for (int b = 0; b < kGemvDepth - 1; ++b)
            if (b < ws.nbatch) load_batch<FMT>(p, ws, b, e, wbase, sbase, j, units, wbuf[b], sbuf[b]);
        __syncthreads();
        stage_activations<FMT, ACT>(p, smem, row0, c0, mc);
        __syncthreads();
        for (int q = 0; q < ws.nbatch; q += kGemvDepth) {
#pragma unroll
            for (int i = 0; i < kGemvDepth; ++i) {
                const int qq = q + i;
                if (qq + kGemvDepth - 1 < ws.nbatch)
                    load_batch<FMT>(p, ws, qq + kGemvDepth - 1, e, wbase, sbase, j, units,
                                    wbuf[(i + kGemvDepth - 1) % kGemvDepth], sbuf[(i + kGemvDepth - 1) % kGemvDepth]);
                if (qq < ws.nbatch)
                    compute_batch<FMT, ACT, MAXM, PAIR>(p, ws, qq, mat, j, units, smem, row0 + c0, mc, wbuf[i],
                                                        sbuf[i], acc);
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

// LDS for staged activations per workgroup.  Small enough that several workgroups share a
// CU (occupancy matters more than the token tile: decode experts mostly own one row);
// experts with more rows than fit loop over token chunks.
#ifndef MOE_GEMV_LDS_BUDGET
#define MOE_GEMV_LDS_BUDGET (32 * 1024)
#endif
constexpr size_t kGemvLdsBudget = MOE_GEMV_LDS_BUDGET;

moe_status gemv_launch(int fmt, int act, bool pair, GemvParams p, int slots, int max_rows_per_expert,
                       hipStream_t stream, const char *what) {
    const bool act_f32 = act == kActF32;
    const int units = fmt == kFmtMXFP4 ? p.K / 32 : (fmt == kFmtFP8 ? p.K / 16 : p.K / 8);
    pick_layout(units, pair, &p.G, &p.nl);
    const size_t row_lds = (size_t)p.K * (act_f32 ? 4 : 2);
    int fit = (int)(kGemvLdsBudget / row_lds);
    if (fit < 1) fit = (int)(64 * 1024 / row_lds);   // wide rows: one token per chunk
    if (fit < 1) {
        set_error("%s: an activation row of %zu bytes does not fit in LDS", what, row_lds);
        return MOE_ERR_UNSUPPORTED;
    }
    // token chunk: rows per expert that fit, at most the widest register tile (8)
    int want = max_rows_per_expert < fit ? max_rows_per_expert : fit;
    want = want < 1 ? 1 : (want > 8 ? 8 : want);
    int maxm = 1;
    while (maxm < want) maxm *= 2;
    p.chunk = want;
    const int rows_per_pass = pair ? 32 / p.G : 64 / p.G;
    // aim for MOE_GEMV_TARGET_WG workgroups over the whole launch, at least one pass per wave
    long long rows_total = (long long)p.N * slots;
    int rpw = (int)(rows_total / MOE_GEMV_TARGET_WG);
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

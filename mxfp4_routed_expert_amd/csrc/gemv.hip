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
#ifndef MOE_GEMV_TARGET_WAVES
#define MOE_GEMV_TARGET_WAVES 4096  // waves a launch aims for (all resident at once)
#endif
#ifndef MOE_GEMV_THREADS
#define MOE_GEMV_THREADS 256        // threads per workgroup
#endif
#ifndef MOE_GEMV_NT
#define MOE_GEMV_NT 1            // non-temporal weight loads
#endif
#ifndef MOE_GEMV_WAVES_PER_EU
#define MOE_GEMV_WAVES_PER_EU 0  // occupancy hint (0: compiler's choice)
#endif
constexpr int kGemvThreads = MOE_GEMV_THREADS;
constexpr int kGemvUnroll = MOE_GEMV_UNROLL;
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
// bf16).  Rows whose index is out of range are staged as zeros.  The source rows of the
// (at most 8) staged rows are resolved first, then each thread issues its loads in groups
// of kStageU independent loads before storing any, so staging costs a few memory round
// trips rather than one per element.
constexpr int kStageU = 4;

template <int FMT, int ACT>
MOE_DEV void stage_activations(const GemvParams &p, unsigned char *smem, int row0, int c0, int mc) {
    constexpr int ASZ = ACT == kActF32 ? 4 : 2;
    const int K = p.K;
    __shared__ int s_arow[8];
    if (threadIdx.x < 8) {
        const int m = threadIdx.x;
        const int r = row0 + c0 + min(m, mc - 1);
        int a = 0;
        if (p.n_act_rows > 1) {               // one activation row (a single token): no lookup
            a = p.gather ? p.sorted_pairs[r] : r;
            if (p.gather) a = a >= 0 ? a / p.k : -1;
        }
        s_arow[m] = (m < mc && a >= 0 && a < p.n_act_rows) ? a : -1;
    }
    lds_barrier();                         // (weight loads issued before stay in flight)
    auto row_of = [&](int m) { return s_arow[m]; };
    if constexpr (ACT == kActMX) {
        const int nb = K / 32;
        const int total = mc * nb;
        for (int i0 = threadIdx.x; i0 < total; i0 += kGemvThreads * kStageU) {
            u32x4 cv[kStageU];
            uint32_t sb[kStageU];
            int src[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = min(i0 + u * kGemvThreads, total - 1);
                const int m = i / nb, blk = i - m * nb;
                src[u] = row_of(m);
                const int a = max(src[u], 0);
                cv[u] = ((const u32x4 *)((const uint8_t *)p.act + (size_t)a * (K / 2)))[blk];
                sb[u] = p.act_s[(size_t)a * nb + blk];
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kGemvThreads;
                if (i >= total) break;
                const int m = i / nb, blk = i - m * nb;
                u32x4 *dst = (u32x4 *)(smem + ((size_t)m * K + (size_t)blk * 32) * 2);
                const int z = act_swizzle<kFmtMXFP4, false>(blk);
                const bool ok = src[u] >= 0;
                const float sc = e8m0_to_f32(sb[u]);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[u][d], sc, 0);
                    const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[u][d], sc, 1);
                    const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[u][d], sc, 2);
                    const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cv[u][d], sc, 3);
                    const u32x4 val = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                       __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
                    dst[d ^ z] = ok ? val : u32x4{0, 0, 0, 0};
                }
            }
        }
    } else {
        const int act_vec = K * ASZ / 16;      // 16-byte vectors per activation row
        const int total = mc * act_vec;
        constexpr int P = act_slots<FMT, ACT == kActF32>();
        for (int i0 = threadIdx.x; i0 < total; i0 += kGemvThreads * kStageU) {
            u32x4 val[kStageU];
            int src[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = min(i0 + u * kGemvThreads, total - 1);
                const int m = i / act_vec, v = i - m * act_vec;
                src[u] = row_of(m);
                val[u] = ((const u32x4 *)((const unsigned char *)p.act + (size_t)max(src[u], 0) * K * ASZ))[v];
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kGemvThreads;
                if (i >= total) break;
                const int m = i / act_vec, v = i - m * act_vec;
                const int b = v / P, sl = v - b * P;
                ((u32x4 *)smem)[(size_t)m * act_vec + b * P + (sl ^ act_swizzle<FMT, ACT == kActF32>(b))] =
                    src[u] >= 0 ? val[u] : u32x4{0, 0, 0, 0};
            }
        }
    }
}

MOE_DEV void gemv_dma16(const void *src, uint32_t lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

MOE_DEV void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A single activation row (one token) copied to LDS row 0 by direct global->LDS loads, in
// the slot order stage_activations gives it: the swizzle is an XOR, so lane q of the copy
// reads source vector b*P + (q%P ^ z(b)).  Lanes past the row read vector 0 into the padding
// of the last 1 KiB block (the launch rounds the LDS size up to 1 KiB).  Issued before the
// expert lookup, so the two memory round trips overlap; wait_vm_all() before LDS is read.
template <int FMT, int ACT>
MOE_DEV void stage_row_dma(const GemvParams &p, unsigned char *smem) {
    constexpr bool F32 = ACT == kActF32;
    constexpr int P = act_slots<FMT, F32>();
    const int act_vec = p.K * (F32 ? 4 : 2) / 16;
    const int nblk = (act_vec + 63) / 64;
    const int lane = lane_id();
    for (int c = __builtin_amdgcn_readfirstlane(wave_id()); c < nblk; c += kGemvThreads / 64) {
        const int q = c * 64 + lane;
        const int b = q / P, sl = q - b * P;
        const int v = q < act_vec ? b * P + (sl ^ act_swizzle<FMT, F32>(b)) : 0;
        gemv_dma16((const u32x4 *)p.act + v, (uint32_t)(uintptr_t)(smem + (size_t)c * 1024));
    }
}

// wbase / sbase: this lane's matrix (gate or up for the pair), chosen once per kernel with a
// select -- indexing the parameter arrays by a lane-dependent value would load the pointer
// from memory on every use.  Every load is issued unconditionally from a clamped, valid
// address: a load under a branch would make the compiler wait for it (and, loads retiring
// in order, for every load before it) where the branch joins.  Slots past the row or the
// row range are skipped when the batch is consumed.  Scale bytes stay raw until then.
// Batch ib of a pass covers this lane's units i0 .. i0+U-1 of row n (n clamped to a valid row).
// A batch that will not be consumed (live false: the wave has no further pass) is still
// issued, from the first bytes of the arrays, so that the loads of the loop are
// unconditional and the compiler can keep one batch in flight while the previous one is
// consumed; those bytes stay in cache.
template <int FMT>
MOE_DEV void load_batch(const GemvParams &p, int n_row, int n_end, int ib, int e, const uint8_t *wbase,
                        const void *sbase, int j, int units, bool live, u32x4 (&w)[kGemvUnroll],
                        uint32_t (&sc)[kGemvUnroll]) {
    const int i0 = ib * kGemvUnroll;
    const int n = min(n_row, n_end - 1);
    const size_t ridx = live ? (size_t)e * p.N + n : 0;
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
        const int b = live ? min(j + (i0 + u) * p.G, units - 1) : 0;
        const size_t wo = (ridx * (size_t)units + b) * 16;
#if MOE_GEMV_NT
        w[u] = __builtin_nontemporal_load((const u32x4 *)(wbase + wo));
#else
        w[u] = *(const u32x4 *)(wbase + wo);
#endif
        if constexpr (FMT == kFmtMXFP4) {
            sc[u] = ((const uint8_t *)sbase)[ridx * units + b];
        } else if constexpr (FMT == kFmtFP8) {
            const size_t srow = live ? (size_t)e * (p.N / 128) + n / 128 : 0;
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
MOE_DEV void compute_batch(const GemvParams &p, int n, int n_end, int ib, int nb, int mat, int j, int units,
                           const unsigned char *smem, int out_row0, int mc, const u32x4 (&w)[kGemvUnroll],
                           const uint32_t (&sc)[kGemvUnroll], float (&acc)[MAXM]) {
    constexpr bool ACT_F32 = ACT == kActF32;
    constexpr int ASZ = ACT_F32 ? 4 : 2;
    constexpr int EPU = FMT == kFmtMXFP4 ? 32 : (FMT == kFmtFP8 ? 16 : 8);
    const int i0 = ib * kGemvUnroll;
    const bool row_ok = n < n_end;
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
    if (ib != nb - 1) return;
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
__global__ MOE_GEMV_ATTR void gemv_kernel(const GemvParams p0) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = kGemvThreads / 64;

    // the shared-expert slot reads its own weight set over the identity rows
    const bool shared = ROUTED && p0.shared_slot >= 0 && (int)blockIdx.y == p0.shared_slot;
    GemvParams p = p0;
    if (shared) {
        p.w[0] = p0.sw[0];
        p.w[1] = p0.sw[1];
        p.s[0] = p0.ss[0];
        p.s[1] = p0.ss[1];
        p.N = p0.sN;
        p.E = 1;
        p.out = p0.sout;
        p.gather = 0;
        p.residual = nullptr;
    }
    const bool pre = ACT != kActMX && p.n_act_rows == 1;
    if (pre) stage_row_dma<FMT, ACT>(p, smem);
    int e = 0, row0 = 0, M = p.T;
    if (ROUTED && !shared) {
        e = wave_nth_nonempty(p.offsets, p.E, blockIdx.y, &row0, &M);
        if (e < 0 || row0 < 0 || M <= 0 || row0 + M > p.R) {
            if (pre) wait_vm_all();          // no copy into LDS may be left in flight
            return;
        }
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
    if (n_begin >= n_end) {
        if (pre) wait_vm_all();
        return;
    }
    const int passes = (n_end - n_begin + rows_per_pass - 1) / rows_per_pass;
    const int nb = (p.nl + kGemvUnroll - 1) / kGemvUnroll;    // batches per pass
    auto row_of = [&](int pass) { return n_begin + pass * rows_per_pass + grp; };

    // Passes (rows_per_pass rows each) are handed out to the waves of the workgroup one at a
    // time from an LDS counter, so a wave whose loads are served late is not left with a
    // fixed share of the work: the others take more passes.  Each wave starts with pass
    // `wave`, asks for its next pass while loading the current one, and stops at the first
    // pass past the end.  Batches alternate between two register buffers, one in flight
    // while the other is consumed.
    __shared__ int s_pass;
    auto grab = [&](int after) {
        int v = passes;
        if (after < passes) {
            int g = 0;
            if (lane == 0) g = atomicAdd(&s_pass, 1);
            v = min(__builtin_amdgcn_readfirstlane(g), passes);
        }
        return v;
    };
    u32x4 wa[kGemvUnroll], wb[kGemvUnroll];
    uint32_t sa[kGemvUnroll], sb[kGemvUnroll];
    float acc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;

    for (int c0 = 0; c0 < M; c0 += p.chunk) {
        const int mc = min(p.chunk, M - c0);
        lds_barrier();                         // the previous chunk is done with LDS and the counter
        if (threadIdx.x == 0) s_pass = NW;
        int P = min(wave, passes), ib = 0;     // batch being consumed: pass P, batch ib
        // the first weight batch is in flight while the activations are staged
        load_batch<FMT>(p, row_of(P), n_end, 0, e, wbase, sbase, j, units, P < passes, wa, sa);
        if (pre && c0 == 0) wait_vm_all();     // the row copied at entry (and the first batch)
        if (!(pre && mc == 1)) stage_activations<FMT, ACT>(p, smem, row0, c0, mc);
        lds_barrier();
        int Pn = grab(P);                      // the wave's next pass
        int Pnn = passes;
        // one batch: load the following one into `nx`, consume `cu`; false when the wave is done
        auto step = [&](u32x4 (&cu)[kGemvUnroll], uint32_t (&cs)[kGemvUnroll], u32x4 (&nx)[kGemvUnroll],
                        uint32_t (&ns)[kGemvUnroll]) {
            const bool last = ib + 1 == nb;
            const int P2 = last ? Pn : P, ib2 = last ? 0 : ib + 1;
            load_batch<FMT>(p, row_of(P2), n_end, ib2, e, wbase, sbase, j, units, P2 < passes, nx, ns);
            if (last) Pnn = grab(Pn);          // needed one pass later
            compute_batch<FMT, ACT, MAXM, PAIR>(p, row_of(P), n_end, ib, nb, mat, j, units, smem, row0 + c0, mc,
                                                cu, cs, acc);
            if (last) {
                P = Pn;
                Pn = Pnn;
                ib = 0;
            } else {
                ++ib;
            }
            return P < passes;
        };
        bool more = P < passes;
        while (more) {
            more = step(wa, sa, wb, sb);
            if (!more) break;
            more = step(wb, sb, wa, sa);
        }
    }
}

static void pick_layout(int units, bool pair, int *G, int *nl);

// ------------------------------------------------------------------ down + combine
// Decode-sized batches: one workgroup per (range of output rows, token) computes
//   out[t][n] = sum_j tw[t][j] * (W_down[e_j][n] . h_j) + g_t * (W_shared_down[n] . hs_t)
// directly, the k routed slots in order, then the shared expert -- the same sum in the same
// order as the combine step, without writing and re-reading the expert rows.
//   * The token's k+1 float32 h rows are copied into LDS by direct global->LDS loads
//     (unit-swizzled as for the GEMV), waited for before the first weight batches are
//     issued (behind them the copy would land much later).
//   * A lane group of G lanes covers kDcRows rows of one slot: every h value read from LDS
//     serves kDcRows weight rows (a float32 h costs 8x the LDS bytes of the FP4 weights it
//     multiplies, so one row per read would make LDS, not HBM, the limit).
//   * Work items are (pass of 64/G * kDcRows rows, slot); wave w takes items w, w+8, ...
//     and keeps kDcDepth batches of loads in flight.  Each item's dot products go to an
//     LDS table part[slot][row]; after a barrier every row's output is the slot-ordered
//     sum of its table column.
#ifndef MOE_DM_ROUND
#define MOE_DM_ROUND 4           // MXFP4 (matrix-core) path: rows per workgroup rounded to this (tiles of 16 may end past them)
#endif
#ifndef MOE_DC_ROWS
#define MOE_DC_ROWS 4            // weight rows per lane group
#endif
#ifndef MOE_DC_DEPTH
#define MOE_DC_DEPTH 2           // batches in flight per wave
#endif
constexpr int kDcRows = MOE_DC_ROWS;
constexpr int kDcDepth = MOE_DC_DEPTH;
static_assert((64 / 4) * kDcRows <= kDcMaxRows, "a pass of the narrowest lane groups must fit the table");

MOE_DEV void dc_dma16(const void *src, uint32_t lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// s[r] = unscaled dot product of weight unit w[r] (row r) with the float32 activations of
// the unit in LDS (slots swizzled with key z); each activation vector is read once.
template <int FMT, int R>
MOE_DEV void unit_dot_rows(const u32x4 (&w)[R], const float *a_unit, int z, float (&s)[R]) {
    const f32x4 *a4s = (const f32x4 *)a_unit;
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.0f;
    if constexpr (FMT == kFmtMXFP4) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x4 lo = a4s[(2 * d) ^ z], hi = a4s[(2 * d + 1) ^ z];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const f32x2 w0 = fp4x2_to_f32x2<0>(w[r][d]), w1 = fp4x2_to_f32x2<1>(w[r][d]);
                const f32x2 w2 = fp4x2_to_f32x2<2>(w[r][d]), w3 = fp4x2_to_f32x2<3>(w[r][d]);
                float v = s[r];
                v = fmaf(w0.x, lo[0], v); v = fmaf(w0.y, lo[1], v);
                v = fmaf(w1.x, lo[2], v); v = fmaf(w1.y, lo[3], v);
                v = fmaf(w2.x, hi[0], v); v = fmaf(w2.y, hi[1], v);
                v = fmaf(w3.x, hi[2], v); v = fmaf(w3.y, hi[3], v);
                s[r] = v;
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x4 av = a4s[d ^ z];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const f32x2 w0 = fp8x2_to_f32x2<false>(w[r][d]), w1 = fp8x2_to_f32x2<true>(w[r][d]);
                float v = s[r];
                v = fmaf(w0.x, av[0], v); v = fmaf(w0.y, av[1], v);
                v = fmaf(w1.x, av[2], v); v = fmaf(w1.y, av[3], v);
                s[r] = v;
            }
        }
    }
}

// Position of a wave's batch: item (pass, slot j), sub-batch ib; every field wave-uniform.
struct DcPos {
    int q, j, ib, pass;
};

template <int FMT, int U>
__global__ __launch_bounds__(kDcThreads) void down_combine_kernel(const DownCombineParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_e[MOE_MAX_TOPK + 1], s_r[MOE_MAX_TOPK + 1];
    __shared__ float s_w[MOE_MAX_TOPK + 1];
    constexpr int NW = kDcThreads / 64;
    constexpr int R = kDcRows;
    constexpr int EPU = FMT == kFmtMXFP4 ? 32 : 16;
    constexpr int P = act_slots<FMT, true>();
    using ScT = typename std::conditional<FMT == kFmtMXFP4, uint8_t, uint32_t>::type;
    const int t = blockIdx.y;
    const int nslot = p.k + (p.sw ? 1 : 0);
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    if (tid < nslot) {
        int e = 0, r = t;
        float wt = p.sg ? p.sg[t] : 1.0f;
        if (tid < p.k) {
            const int pi = t * p.k + tid;
            e = p.ids[pi];
            r = p.p2r[pi];
            wt = p.tw[pi];
            if (e < 0 || e >= p.E || r < 0 || r >= p.R) {      // dropped pair: contributes 0
                e = r = -1;
                wt = 0.0f;
            }
        }
        s_e[tid] = e;
        s_r[tid] = r;
        s_w[tid] = wt;
    }
    __syncthreads();

    const int units = units_per_row<FMT>(p.I);
    const int G = p.G, grp = lane / G, jl = lane & (G - 1);
    const int rpp = (64 / G) * R;                          // rows per pass
    const int nb = (p.nl + U - 1) / U;
    const int n_begin = blockIdx.x * p.rows_per_wg;
    const int n_end = min(p.N, n_begin + p.rows_per_wg);
    if (n_begin >= n_end) return;                          // the whole workgroup
    const int npass = (n_end - n_begin + rpp - 1) / rpp;
    const int nitems = npass * nslot;
    const int my_items = wave < nitems ? (nitems - 1 - wave) / NW + 1 : 0;
    const int nq = my_items * nb;
    const size_t row_bytes = FMT == kFmtMXFP4 ? (size_t)p.I / 2 : (size_t)p.I;
    const int act_vec = p.I / 4;                           // 16-byte vectors per float32 row
    float *part = (float *)(smem + p.h_lds_bytes);          // [nslot][rows_per_wg]

    auto advance = [&](DcPos &c) {
        ++c.q;
        if (++c.ib == nb) {
            c.ib = 0;
            c.j += NW;
            while (c.j >= nslot) {
                c.j -= nslot;
                ++c.pass;
            }
        }
    };
    // rows of the lane group in a pass: pass * rpp + grp * R + r
    auto load = [&](const DcPos &c, u32x4 (&w)[U][R], ScT (&sc)[U][R]) {
        const bool sh = c.j >= p.k;
        const int e = sh ? 0 : max(__builtin_amdgcn_readfirstlane(s_e[c.j]), 0);
        const uint8_t *wb = sh ? p.sw : p.w;
        const void *sb = sh ? p.ss : p.s;
        const int n0 = n_begin + c.pass * rpp + grp * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(n0 + r, n_end - 1);
            const size_t ridx = (size_t)e * p.N + n;
            const uint8_t *wrow = wb + ridx * row_bytes;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int b = min(jl + (c.ib * U + u) * G, units - 1);
                w[u][r] = __builtin_nontemporal_load((const u32x4 *)(wrow + (size_t)b * 16));
                if constexpr (FMT == kFmtMXFP4) {
                    sc[u][r] = ((const uint8_t *)sb)[ridx * units + b];
                } else {
                    const size_t srow = (size_t)e * (p.N / 128) + n / 128;
                    sc[u][r] = __float_as_uint(((const float *)sb)[srow * (p.I / 128) + (b * 16) / 128]);
                }
            }
        }
    };
    float dot[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dot[r] = 0.0f;
    // Batch at c into dot (branch-free: out-of-row units are computed on a clamped unit and
    // discarded by a select); the item's last sub-batch reduces over the lane group and
    // stores the rows' dot products for slot j (0 for a dropped pair).  Positions past the
    // wave's last batch compute on reloaded data and store nothing.
    auto compute = [&](const DcPos &c, const u32x4 (&w)[U][R], const ScT (&sc)[U][R]) {
        const float *hrow = (const float *)smem + (size_t)c.j * p.I;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = jl + (c.ib * U + u) * G;
            const int bc = min(b, units - 1);
            float s[R];
            unit_dot_rows<FMT, R>(w[u], hrow + (size_t)bc * EPU, act_swizzle<FMT, true>(bc), s);
            const bool ok = (c.ib * U + u) < p.nl && b < units;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v = fmaf(s[r], unit_scale_value(FMT, (uint32_t)sc[u][r]), dot[r]);
                dot[r] = ok ? v : dot[r];
            }
        }
        if (c.ib != nb - 1) return;
        const bool drop = __builtin_amdgcn_readfirstlane(s_e[c.j]) < 0;
        const int l0 = c.pass * rpp + grp * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float v = group_sum(dot[r], G);
            dot[r] = 0.0f;
            if (drop) v = 0.0f;
            if (jl == 0 && c.q < nq && n_begin + l0 + r < n_end) part[c.j * p.rows_per_wg + l0 + r] = v;
        }
    };

    // first batches in flight before the h copy
    u32x4 wv[kDcDepth][U][R];
    ScT sv[kDcDepth][U][R];
    // h rows -> LDS: position i = (slot j, vector v) holds vector b*P + (s ^ swz(b)) of the
    // slot's row, v = b*P + s; invalid slots copy row 0 (never used).  The copy covers whole
    // 64-vector blocks; the tail of the last block reads a valid vector into the padding.
    // It is waited for before the first weight loads are issued, so it is not queued behind
    // them.
    {
        const int total = nslot * act_vec;
        const int blocks = (total + 63) / 64;
        for (int blk = wave; blk < blocks; blk += NW) {
            const int i = min(blk * 64 + lane, total - 1);
            const int j = i / act_vec, v = i - j * act_vec;
            const int b = v / P, sl = v - b * P;
            const int vs = b * P + (sl ^ act_swizzle<FMT, true>(b));
            const float *row = j < p.k ? p.h + (size_t)max(s_r[j], 0) * p.I : p.hs + (size_t)t * p.I;
            dc_dma16(row + (size_t)vs * 4, (uint32_t)(uintptr_t)(smem + (size_t)blk * 1024));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    DcPos lp{0, wave % nslot, 0, wave / nslot};
    const DcPos first = lp;
    if (nq > 0) {
#pragma unroll
        for (int d = 0; d < kDcDepth; ++d) {
            load(lp, wv[d], sv[d]);
            if (lp.q < nq - 1) advance(lp);
        }
    }

    DcPos cp = first;
    const int nqr = (nq + kDcDepth - 1) / kDcDepth * kDcDepth;
    for (int q0 = 0; q0 < nqr; q0 += kDcDepth) {
#pragma unroll
        for (int d = 0; d < kDcDepth; ++d) {
            compute(cp, wv[d], sv[d]);
            advance(cp);
            load(lp, wv[d], sv[d]);
            if (lp.q < nq - 1) advance(lp);
        }
    }
    __syncthreads();
    for (int lr = tid; lr < n_end - n_begin; lr += kDcThreads) {
        float acc = 0.0f;
        for (int j = 0; j < nslot; ++j) acc = fmaf(s_w[j], part[j * p.rows_per_wg + lr], acc);   // slot order
        p.out[(size_t)t * p.N + n_begin + lr] = acc;
    }
}

// LDS of a down-combine workgroup: the slots' h (4 * dc_plane_ld(I) bytes each), padded
// to whole 1 KiB copy blocks, then the [slots][kDcMaxRows] float table.
size_t down_combine_lds(int k, bool shared, int I) {
    const size_t nslot = (size_t)k + (shared ? 1 : 0);
    return align_up(nslot * 4 * dc_plane_ld(I), 1024) + nslot * kDcMaxRows * 4;
}

template <int FMT>
static void (*down_combine_fn(int U))(const DownCombineParams) {
    switch (U) {
        case 1: return down_combine_kernel<FMT, 1>;
        case 2: return down_combine_kernel<FMT, 2>;
        case 3: return down_combine_kernel<FMT, 3>;
        case 4: return down_combine_kernel<FMT, 4>;
        default: return down_combine_kernel<FMT, 5>;
    }
}

// Units per lane per batch for nl units per lane: the U <= 5 (larger batches of kDcRows
// rows do not fit the registers) that wastes the fewest loads, the larger on a tie.
static int down_combine_batch(int nl) {
    int best = 1, waste = INT_MAX;
    for (int u = 1; u <= 5; ++u) {
        const int w = (nl + u - 1) / u * u - nl;
        if (w <= waste) {
            best = u;
            waste = w;
        }
    }
    return best;
}

moe_status down_combine_launch(int fmt, DownCombineParams p, hipStream_t stream) {
    const bool mfma = fmt == kFmtMXFP4;
    const int units = fmt == kFmtMXFP4 ? p.I / 32 : p.I / 16;
    int U = 1, rpp = MOE_DM_ROUND;                         // MFMA path: 16-row tiles, the last one clamped

    if (!mfma) {
        // 16 lanes per row segment while a lane still gets >= 4 units; short rows use the
        // GEMV layout
        p.G = 16;
        p.nl = (units + 15) / 16;
        if (p.nl < 4) pick_layout(units, false, &p.G, &p.nl);
        U = down_combine_batch(p.nl);
        rpp = (64 / p.G) * kDcRows;
    }
    // about one workgroup per CU in total (LDS holds k+1 rows of h; an HBM-bound launch
    // does not need every CU), whole passes, at most kDcMaxRows rows
    const long long rows_total = (long long)p.N * p.T;
    int rpw = (int)((rows_total + 255) / 256);
    rpw = (max(rpw, rpp) + rpp - 1) / rpp * rpp;
    rpw = min(rpw, max(rpp, kDcMaxRows / rpp * rpp));
    p.rows_per_wg = rpw;
    const int nslot = p.k + (p.sw ? 1 : 0);
    p.h_lds_bytes = (int)align_up((size_t)nslot * 4 * dc_plane_ld(p.I), 1024);
    const size_t lds = down_combine_lds(p.k, p.sw != nullptr, p.I);
    dim3 grid((p.N + rpw - 1) / rpw, p.T);
    if (mfma) {
        down_combine_mfma_launch(p, grid, lds, stream);
    } else {
        hipLaunchKernelGGL(down_combine_fn<kFmtFP8>(U), grid, dim3(kDcThreads), lds, stream, p);
    }
    return launch_check("moe_expert_down_combine");
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
    // aim for at most MOE_GEMV_TARGET_WAVES waves over the whole launch (rounding the rows
    // per workgroup up: a workgroup more than the target puts a fifth one on some CUs, whose
    // workgroups then finish last), at least one pass per wave
    const int n_grid = p.shared_slot >= 0 ? max(p.N, p.sN) : p.N;
    const long long rows_total = (long long)n_grid * slots;
    const int target_wgs = MOE_GEMV_TARGET_WAVES / (kGemvThreads / 64);
    int rpw = (int)((rows_total + target_wgs - 1) / target_wgs);
    const int min_rpw = rows_per_pass * (kGemvThreads / 64);
    if (rpw < min_rpw) rpw = min_rpw;
    rpw = (rpw + rows_per_pass - 1) / rows_per_pass * rows_per_pass;
    p.rows_per_wg = rpw;
    dim3 grid((n_grid + rpw - 1) / rpw, slots);
    const size_t lds = align_up((size_t)p.chunk * row_lds, 1024);   // whole 1 KiB blocks: stage_row_dma
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

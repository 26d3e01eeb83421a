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
#include <algorithm>
#include <mutex>

#include "dm_body.h"
#include "gemv.h"
#include "router_row.h"
#include "step_sync.h"
#include "topk.h"

namespace moe {

constexpr int kGemvThreads = 256;          // threads per workgroup (per-expert GEMV)
// ... with wide activation rows (see gemv_launch): 16 waves for bf16 activations, 8 for
// float32 ones, whose dot products read twice the LDS bytes and hold more registers
template <int ACT>
constexpr int gemv_wide_threads() { return ACT == kActF32 ? 512 : 1024; }
constexpr int kGemvUnroll = 4;             // 16-byte weight loads issued per lane per batch
constexpr int kGemvTargetWaves = 4096;     // waves a launch aims for (all resident at once)

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

template <int FMT, int ACT, int THREADS>
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
        for (int i0 = threadIdx.x; i0 < total; i0 += THREADS * kStageU) {
            u32x4 cv[kStageU];
            uint32_t sb[kStageU];
            int src[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = min(i0 + u * THREADS, total - 1);
                const int m = i / nb, blk = i - m * nb;
                src[u] = row_of(m);
                const int a = max(src[u], 0);
                cv[u] = ((const u32x4 *)((const uint8_t *)p.act + (size_t)a * (K / 2)))[blk];
                sb[u] = p.act_s[(size_t)a * nb + blk];
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * THREADS;
                if (i >= total) break;
                const int m = i / nb, blk = i - m * nb;
                u32x4 *dst = (u32x4 *)(smem + ((size_t)m * K + (size_t)blk * 32) * 2);
                const int z = act_swizzle<kFmtMXFP4, false>(blk);
                const bool ok = src[u] >= 0;
                const float sc = e8m0_to_f32(sb[u]);
#pragma unroll
                for (int d = 0; d < 4; ++d) dst[d ^ z] = ok ? fp4x8_scaled_bf16_bits(cv[u][d], sc) : u32x4{0, 0, 0, 0};
            }
        }
    } else {
        const int act_vec = K * ASZ / 16;      // 16-byte vectors per activation row
        const int total = mc * act_vec;
        constexpr int P = act_slots<FMT, ACT == kActF32>();
        for (int i0 = threadIdx.x; i0 < total; i0 += THREADS * kStageU) {
            u32x4 val[kStageU];
            int src[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = min(i0 + u * THREADS, total - 1);
                const int m = i / act_vec, v = i - m * act_vec;
                src[u] = row_of(m);
                val[u] = ((const u32x4 *)((const unsigned char *)p.act + (size_t)max(src[u], 0) * K * ASZ))[v];
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * THREADS;
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
template <int FMT, int ACT, int THREADS>
MOE_DEV void stage_row_dma(const GemvParams &p, unsigned char *smem) {
    constexpr bool F32 = ACT == kActF32;
    constexpr int P = act_slots<FMT, F32>();
    const int act_vec = p.K * (F32 ? 4 : 2) / 16;
    const int nblk = (act_vec + 63) / 64;
    const int lane = lane_id();
    for (int c = __builtin_amdgcn_readfirstlane(wave_id()); c < nblk; c += THREADS / 64) {
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
        w[u] = __builtin_nontemporal_load((const u32x4 *)(wbase + wo));
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

template <int FMT, int ACT, int MAXM, bool PAIR, bool ROUTED, int THREADS>
__global__ __launch_bounds__(THREADS) void gemv_kernel(const GemvParams p0) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = THREADS / 64;

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
    if (pre) stage_row_dma<FMT, ACT, THREADS>(p, smem);
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
        if (!(pre && mc == 1)) stage_activations<FMT, ACT, THREADS>(p, smem, row0, c0, mc);
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

// ------------------------------------------------------------------ flat schedule
// Decode-sized launches (at most kFlatMaxTok float or bf16 activation rows): one workgroup of
// kFlatThreads threads per CU.  The launch's work is a list of passes -- rows_per_pass matrix
// rows of one slot for up to MAXM of the slot's rows -- slot after slot, where a slot is a
// routed expert that owns rows (in expert order) or the fused shared expert.  Workgroup b
// takes the b-th of gridDim.x equal contiguous ranges of the list, and its waves take passes
// from that range one at a time through an LDS counter.  (With several workgroups per CU the
// oldest one's waves win the issue arbitration, and the youngest finishes last with a quarter
// of the CU's loads in flight; one workgroup per CU keeps every wave streaming until the CU's
// share is done.)  Every activation row is staged once per workgroup by direct global->LDS
// copies, and the slot table -- expert, first row, rows, first pass -- is built once per
// workgroup from expert_offsets while those copies are in flight.
constexpr int kFlatThreads = 1024;
constexpr int kFlatMaxTok = 8;            // activation rows staged: all of the launch's rows
constexpr int kFlatMaxSlots = 256;        // routed rows (<= kFlatMaxSlots - 1) plus the shared slot
constexpr size_t kFlatLdsBudget = 96 * 1024;

// (by waves first_wave .. the last; the caller's wave is one of them)
template <int FMT, int ACT>
MOE_DEV void stage_rows_dma(const GemvParams &p, unsigned char *smem, int rs, int first_wave) {
    constexpr bool F32 = ACT == kActF32;
    constexpr int P = act_slots<FMT, F32>();
    const int act_vec = p.K * (F32 ? 4 : 2) / 16;
    const int nblk = (act_vec + 63) / 64;
    const int lane = lane_id();
    for (int c = __builtin_amdgcn_readfirstlane(wave_id()) - first_wave; c < p.n_act_rows * nblk;
         c += kFlatThreads / 64 - first_wave) {
        const int m = c / nblk, cb = c - m * nblk;
        const int q = cb * 64 + lane;
        const int b = q / P, sl = q - b * P;
        const int v = q < act_vec ? b * P + (sl ^ act_swizzle<FMT, F32>(b)) : 0;
        const u32x4 *row = (const u32x4 *)((const unsigned char *)p.act + (size_t)m * p.K * (F32 ? 4 : 2));
        gemv_dma16(row + v, (uint32_t)(uintptr_t)(smem + (size_t)m * rs + (size_t)cb * 1024));
    }
}

// b * total / nb: the start of workgroup b's equal share of `total` items.  In 32-bit unsigned
// arithmetic when the product fits (a 64-bit division is a long software routine, and this
// one sits on the routing's critical path).
MOE_DEV int share_begin(int b, int total, int nb) {
    const uint64_t prod = (uint64_t)(uint32_t)b * (uint32_t)total;
    if (prod <= 0xffffffffull) return (int)((uint32_t)prod / (uint32_t)nb);
    return (int)(prod / (uint32_t)nb);
}

// A pass resolved to its slot: wave-uniform fields, plus this lane's matrix row n, the row's
// index in the stacked matrix and its scale row.
struct FlatPass {
    int e, N, r0, m0, mc, n;
    bool sh, live;
    size_t ridx, srow;
    const uint8_t *wb;
    const void *sb;
};

// Pass P -> its slot and rows.  Scalars are passed one by one: with a struct of them the
// compiler turns a select between two fields into a load from a selected field address,
// and the struct then stays in scratch memory.
template <int FMT, int MAXM>
MOE_DEV FlatPass flat_resolve(int P, int end, int ns, int pN, int sN, int rpp, int grp, const uint8_t *w_r,
                              const void *s_rt, const uint8_t *w_s, const void *s_s, int &cursor, const int *s_e,
                              const int *s_r0, const int *s_m, const int *s_pass0) {
    FlatPass f;
    f.live = P < end;
    if (!f.live) {                                         // no pass: loads read row 0, nothing is stored
        f.e = f.r0 = f.m0 = f.mc = f.n = 0;
        f.N = pN;
        f.sh = false;
        f.ridx = f.srow = 0;
        f.wb = w_r;
        f.sb = s_rt;
        return f;
    }
    int cur = cursor;
    while (cur + 1 < ns && s_pass0[cur + 1] <= P) ++cur;
    const int sl = __builtin_amdgcn_readfirstlane(cur);
    cursor = sl;
    const int e = __builtin_amdgcn_readfirstlane(s_e[sl]);
    f.sh = e < 0;
    f.e = f.sh ? 0 : e;
    f.N = f.sh ? sN : pN;
    f.r0 = __builtin_amdgcn_readfirstlane(s_r0[sl]);
    const int M = __builtin_amdgcn_readfirstlane(s_m[sl]);
    const int rpc = max((f.N + rpp - 1) / rpp, 1);
    const int local = P - __builtin_amdgcn_readfirstlane(s_pass0[sl]);
    const int mch = local / rpc;
    f.m0 = mch * MAXM;
    f.mc = min(MAXM, M - f.m0);
    f.n = (local - mch * rpc) * rpp + grp;
    const int nc = min(f.n, f.N - 1);
    f.ridx = (size_t)f.e * f.N + nc;
    f.srow = FMT == kFmtFP8 ? (size_t)f.e * (f.N / 128) + nc / 128 : 0;
    f.wb = f.sh ? w_s : w_r;
    f.sb = f.sh ? s_s : s_rt;
    return f;
}

constexpr int kFlatTopkNK = 8;             // routing in the prologue: E <= 64 * kFlatTopkNK

// Wait (bounded, sleeping) until an LDS counter reaches v.  Read through an LDS pointer: a
// generic volatile read is a flat load, and its wait would also wait for every global load
// in flight.  The bound only keeps a fault elsewhere from turning into a hang.
MOE_DEV void lds_wait_at_least(int *ctr, int v) {
    volatile __attribute__((address_space(3))) int *c = (volatile __attribute__((address_space(3))) int *)ctr;
    for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__builtin_amdgcn_readfirstlane(*c) >= v) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");                         // no LDS read moves above the wait
}

// ROUTE: the routing-in-the-prologue form (p.route): wave t < T selects token t's experts
// (topk_select, the route kernel's selection), and wave 0 builds the slot table of the routed
// experts and the rows' tokens from the selections in the permutation's order (expert, then
// pair); workgroup 0 also writes the routing results and the permutation.  The shared expert
// does not depend on the routing: the other waves copy the activation rows and take the
// workgroup's share of the shared expert's passes (an equal contiguous range of them) while
// the routing runs, and every wave takes routed passes once wave 0 has published the table.
// Waves hand over through LDS counters, not workgroup barriers, so none holds the others
// back.
//
// STEP (with ROUTE): the gate/up phase of the single-launch decode step (decode_step_kernel):
// the routing waves first collect every workgroup's logits (step_get_logits), the
// workgroup's routing is also kept in sc->lds for the down phase, h is stored at device
// scope (step_put) and every wave waits for its h stores before it returns.
template <int FMT, int ACT, int MAXM, bool PAIR, bool ROUTE, bool STEP>
MOE_DEV void flat_body(const GemvParams &p, const StepCtx *sc) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_sid[ROUTE ? 64 : 1];
    __shared__ int s_e[kFlatMaxSlots], s_r0[kFlatMaxSlots], s_m[kFlatMaxSlots], s_pass0[kFlatMaxSlots + 1];
    __shared__ int s_tok[kFlatMaxSlots];
    __shared__ int s_ns, s_beg, s_end, s_next, s_perm;
    // ROUTE: the shared slot as a one-entry table, its pass counter and the hand-off counters
    __shared__ int s_she[1], s_shr0[1], s_shm[1], s_shpass0[2];
    __shared__ int s_shnext, s_dma, s_topk, s_tab;
    constexpr int NW = kFlatThreads / 64;
    constexpr bool F32 = ACT == kActF32;
    constexpr int ASZ = F32 ? 4 : 2;
    constexpr int EPU = FMT == kFmtMXFP4 ? 32 : (FMT == kFmtFP8 ? 16 : 8);
    // units per lane and batch (batches of 8 with two passes in flight measured slower)
    constexpr int U = 4;
    constexpr int SD = U / 4;                              // scale dwords per lane and batch (MXFP4)
    constexpr int NSC = FMT == kFmtMXFP4 ? SD : U;         // scale registers per batch
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    // parameters in locals (a lambda that captures the parameter block by reference can make
    // the compiler keep it in scratch memory and read its fields through pointers)
    const int K = p.K, pN = p.N, sN = p.sN, E = p.E, R = p.R, T = p.T, kk = p.k, nl = p.nl, G = p.G;
    const int n_act = p.n_act_rows;
    const bool routed = p.offsets != nullptr, gather = p.gather != 0, has_sh = p.shared_slot >= 0;
    const int32_t *offsets = p.offsets, *sorted = p.sorted_pairs;
    float *out = p.out, *sout = p.sout;
    const float *residual = p.residual;
    const int rs = (K * ASZ + 1023) / 1024 * 1024;         // LDS bytes per staged row
    const int rpp = PAIR ? 32 / G : 64 / G;
    const int units = units_per_row<FMT>(K);
    const RouteArgs ra = p.route;
    const int T0 = ROUTE ? T : 0;                          // waves that route (and copy no rows)
    int sh_end = 0;
    if constexpr (ROUTE) {
        // the shared slot's passes (rows 0 .. T-1) and this workgroup's equal share of them
        const int S = has_sh ? ((T + MAXM - 1) / MAXM) * ((sN + rpp - 1) / rpp) : 0;
        const int b = blockIdx.x, nb = gridDim.x;
        sh_end = share_begin(b + 1, S, nb);
        if (threadIdx.x == 0) {
            s_she[0] = -1;
            s_shr0[0] = 0;
            s_shm[0] = T;
            s_shpass0[0] = 0;
            s_shpass0[1] = S;
            s_shnext = share_begin(b, S, nb);
            s_dma = s_topk = s_tab = s_perm = 0;
        }
        __syncthreads();
    }
    if (wave >= T0) stage_rows_dma<FMT, ACT>(p, smem, rs, T0);
    if constexpr (ROUTE) {
        if (wave >= T) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's row copies are in LDS
            if (lane == 0) atomicAdd(&s_dma, 1);
        }
        if (wave < T) {
            // the selection is on every workgroup's critical path: it goes first at issue
            __builtin_amdgcn_s_setprio(3);
            const float *lt = ra.logits + (size_t)wave * ra.rows;
            if constexpr (STEP) {
                step_get_logits(sc->sync, sc->tag, wave, ra.rows, sc->lds->lt[wave]);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                lt = sc->lds->lt[wave];
            }
            double *gk = (double *)(smem + (size_t)n_act * rs) + (size_t)wave * E;   // group-limited keys
            const TopkLane r = topk_select<kFlatTopkNK>(lt, E, kk, ra.score, ra.renorm,
                                                        ra.scaling, ra.lbias, ra.sbias, ra.has_sg, gk, ra.n_group,
                                                        ra.topk_group);
            if (lane < kk) {
                s_sid[wave * kk + lane] = r.e;            // -1 when fewer than k keys compare
                if (blockIdx.x == 0) {
                    ra.ids[wave * kk + lane] = r.e;
                    ra.tw[wave * kk + lane] = r.w;
                }
            }
            if (blockIdx.x == 0 && ra.has_sg && lane == 0) ra.sg[wave] = r.sg;
            if constexpr (STEP) {
                if (lane < kk) {
                    sc->lds->ids[wave * kk + lane] = r.e;
                    sc->lds->tw[wave * kk + lane] = r.w;
                }
                if (lane == 0) sc->lds->sg[wave] = r.sg;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // s_sid holds this token's experts
            if (lane == 0) atomicAdd(&s_topk, 1);
            if (wave != 0) __builtin_amdgcn_s_setprio(0);        // (wave 0 builds the table next)
        }
    }

    if (wave == 0) {
        // slots: the experts that own a valid range of rows, in expert order, then the shared
        // expert (e = -1) over the identity rows
        int ns = 0;
        int fast_base = -1;                                // the one-token table's pass count
        if constexpr (ROUTE) {
            lds_wait_at_least(&s_topk, T);
            if (T == 1) {
                // one token: its k experts are distinct, each a slot of one row whose index is the
                // expert's rank among them; pass offsets are multiples of the passes per slot (the
                // table the general form below builds, without its scans)
                const int e = lane < kk ? s_sid[lane] : -1;
                int row = 0;
                for (int q = 0; q < kk; ++q) {
                    const int eq = __builtin_amdgcn_readlane(e, q);
                    row += (eq >= 0 && eq < e) ? 1 : 0;
                }
                if (e >= 0) {
                    s_tok[row] = 0;
                    s_e[row] = e;
                    s_r0[row] = row;
                    s_m[row] = 1;
                }
                if constexpr (STEP) {
                    if (lane < kk) sc->lds->p2r[lane] = e >= 0 ? row : -1;
                }
                ns = __popcll(__ballot(e >= 0));
                const int pps = (pN + rpp - 1) / rpp;
                if (lane < ns) s_pass0[lane] = lane * pps;
                fast_base = ns * pps;
            } else {
                // pair q = (token q / k, slot q % k) -> row = pairs of lower experts + earlier pairs
                // of its expert; the first pair of an expert opens its slot
                // (pair q's expert read from lane q's register: a loop of LDS reads waits out each
                // read's latency in turn)
                const int P = T * kk;
                const int e = lane < P ? s_sid[lane] : -1;
                int row = 0, cnt = 0;
                bool first = e >= 0;
                for (int q = 0; q < P; ++q) {
                    const int eq = __builtin_amdgcn_readlane(e, q);
                    row += (eq >= 0 && (eq < e || (eq == e && q < lane))) ? 1 : 0;
                    cnt += eq == e ? 1 : 0;
                    first = first && !(eq == e && q < lane);
                }
                const uint64_t fm = __ballot(first);
                int slot = 0;
                for (int q = 0; q < P; ++q) slot += (((fm >> q) & 1ull) && __builtin_amdgcn_readlane(e, q) < e) ? 1 : 0;
                if (e >= 0) s_tok[row] = lane / kk;
                if constexpr (STEP) {
                    if (lane < P) sc->lds->p2r[lane] = e >= 0 ? row : -1;
                }
                if (first) {
                    s_e[slot] = e;
                    s_r0[slot] = row;
                    s_m[slot] = cnt;
                }
                ns = __popcll(fm);
            }
        } else if (routed) {
            int o[kMaxOffsetChunks];
#pragma unroll
            for (int c = 0; c < kMaxOffsetChunks; ++c) o[c] = gload_i32(offsets + min(c * 64 + lane, E));
#pragma unroll
            for (int c = 0; c < kMaxOffsetChunks; ++c) {
                if (c * 64 >= E) break;
                const int next = c + 1 < kMaxOffsetChunks ? __shfl(o[c + 1], 0, kWave) : 0;
                int o1 = __shfl_down(o[c], 1, kWave);
                if (lane == 63) o1 = next;
                const int e = c * 64 + lane;
                const bool ne = e < E && o1 > o[c] && o[c] >= 0 && o1 <= R;
                const uint64_t mk = __ballot(ne);
                const int at = ns + __popcll(mk & ((1ull << lane) - 1ull));
                if (ne && at < kFlatMaxSlots - 1) {
                    s_e[at] = e;
                    s_r0[at] = o[c];
                    s_m[at] = o1 - o[c];
                }
                ns += __popcll(mk);
            }
            ns = min(ns, kFlatMaxSlots - 1);
        } else {
            if (lane == 0) {
                s_e[0] = 0;
                s_r0[0] = 0;
                s_m[0] = T;
            }
            ns = 1;
        }
        if (!ROUTE && has_sh) {
            if (lane == 0) {
                s_e[ns] = -1;
                s_r0[ns] = 0;
                s_m[ns] = T;
            }
            ++ns;
        }
        // first pass of each slot: exclusive prefix of ceil(rows / MAXM) * ceil(N / rpp)
        int base = fast_base >= 0 ? fast_base : 0;
        for (int c = 0; fast_base < 0 && c < ns; c += 64) {
            const int sl = c + lane;
            int cnt = 0;
            if (sl < ns) {
                const int N = s_e[sl] < 0 ? sN : pN;
                cnt = (s_m[sl] + MAXM - 1) / MAXM * ((N + rpp - 1) / rpp);
            }
            int inc = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(inc, d, kWave);
                if (lane >= d) inc += v;
            }
            if (sl < ns) s_pass0[sl] = base + inc - cnt;
            base += __shfl(inc, 63, kWave);
        }
        if (lane == 0) {
            s_pass0[ns] = base;
            s_ns = ns;
            const int b = blockIdx.x, nb = gridDim.x;
            const int beg = share_begin(b, base, nb), end = share_begin(b + 1, base, nb);
            s_beg = beg;
            s_end = end;
            s_next = ROUTE ? beg : beg + NW;
        }
        if constexpr (ROUTE) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the table is in LDS
            if (lane == 0) atomicAdd(&s_tab, 1);
            __builtin_amdgcn_s_setprio(0);
        }
    } else if (!ROUTE && wave == 1) {
        // activation row of each routed row (or identity row): -1 when out of range
        const int Rr = routed ? R : T;
        for (int r = lane; r < Rr && r < kFlatMaxSlots; r += 64) {
            int a = r;
            if (routed && gather) {
                a = gload_i32(sorted + r);
                a = a >= 0 ? a / kk : -1;
            }
            s_tok[r] = (a >= 0 && a < n_act) ? a : -1;
        }
    }
    if constexpr (!ROUTE) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const int grp = PAIR ? (lane & 31) / G : lane / G;
    const int j = lane & (G - 1);
    const int mat = PAIR ? (lane >> 5) : 0;
    const uint8_t *w_r = PAIR && mat ? p.w[1] : p.w[0];
    const void *s_rt = PAIR && mat ? p.s[1] : p.s[0];
    const uint8_t *w_s = has_sh ? (PAIR && mat ? p.sw[1] : p.sw[0]) : w_r;
    const void *s_s = has_sh ? (PAIR && mat ? p.ss[1] : p.ss[0]) : s_rt;
    const int nb = (nl + U - 1) / U;    // batches per pass

    // loads of batch ib of a pass (row ridx of the stack wb / sb), from clamped valid addresses
    auto load = [&](const uint8_t *wb, const void *sb, size_t ridx, size_t srow, int ib, u32x4 (&w)[U],
                    uint32_t (&sc)[NSC]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = min(j + (ib * U + u) * G, units - 1);
            w[u] = gload16_nt(wb + (ridx * (size_t)units + b) * 16);
            if constexpr (FMT == kFmtMXFP4) {
                // SD dwords of scales per lane and batch: load k of lane j of the group holds the
                // bytes of units 4(ib*SD*G + k*G + j) .. +3; compute() picks each unit's byte
                if (u < SD) {
                    const int dw = min(ib * SD * G + u * G + j, units / 4 - 1);
                    sc[u] = gload_u32((const uint8_t *)sb + ridx * units + 4 * dw);
                }
            } else if constexpr (FMT == kFmtFP8) {
                sc[u] = gload_u32((const float *)sb + srow * (K / 128) + (b * 16) / 128);
            } else {
                sc[u] = 0;
            }
        }
    };
    float acc[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
    int tok[MAXM];
    auto tokens = [&](const FlatPass &f) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const int r = f.r0 + f.m0 + m;
            const int tk = m < f.mc ? (f.sh ? (f.m0 + m < n_act ? f.m0 + m : -1) : s_tok[min(r, kFlatMaxSlots - 1)]) : -1;
            tok[m] = __builtin_amdgcn_readfirstlane(tk);
        }
    };
    // accumulate batch ib of pass f; after its last batch reduce over the lane group, apply
    // SwiGLU for the pair, write the rows and clear acc
    auto compute = [&](const FlatPass &f, int ib, const u32x4 (&w)[U],
                       const uint32_t (&sc)[NSC]) __attribute__((always_inline)) {
        const bool row_ok = f.n < f.N;
        uint32_t scv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (FMT == kFmtMXFP4) {
                // unit j + G*(U ib + u): byte j%4 of scale dword u/4 of lane (j + G*(u%4))/4
                const uint32_t d = __shfl(sc[u / 4], (lane - j) + ((j + G * (u % 4)) >> 2), kWave);
                scv[u] = (d >> (8 * (j & 3))) & 0xffu;
            } else {
                scv[u] = sc[u];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int b = j + (ib * U + u) * G;
            if (row_ok && (ib * U + u) < nl && b < units) {
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    if (m < f.mc) {
                        const void *a = smem + (size_t)max(tok[m], 0) * rs + (size_t)b * EPU * ASZ;
                        acc[m] = fmaf(unit_dot<FMT, F32>(w[u], a, act_swizzle<FMT, F32>(b)),
                                      unit_scale_value(FMT, scv[u]), acc[m]);
                    }
                }
            }
        }
        if (ib != nb - 1) return;
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
                if (m < f.mc) {
                    float v = tok[m] >= 0 ? acc[m] : 0.0f;
                    if (f.sh) {
                        float *dst = sout + (size_t)(f.m0 + m) * f.N + f.n;
                        if constexpr (STEP) step_put(dst, v);
                        else *dst = v;
                    } else {
                        const size_t o = (size_t)(f.r0 + f.m0 + m) * f.N + f.n;
                        if (residual) v += residual[o];
                        if constexpr (STEP) step_put(out + o, v);
                        else out[o] = v;
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = 0.0f;
    };
    // One phase: passes [.., end) of the routed table (SH false) or of the shared slot's
    // one-entry table (SH true), handed out by that phase's LDS counter; the wave starts at
    // pass P0 (< 0: the counter's next).
    auto run = [&](auto shc, int P0, int end, int ns) __attribute__((always_inline)) {
        constexpr bool SH = decltype(shc)::value;
        // pass P -> its slot; the passes a wave takes only increase, so the slot cursor moves
        // forward
        int cursor = 0;
        auto resolve = [&](int Q) __attribute__((always_inline)) {
            if constexpr (SH)
                return flat_resolve<FMT, MAXM>(Q, end, 1, pN, sN, rpp, grp, w_r, s_rt, w_s, s_s, cursor, s_she, s_shr0,
                                               s_shm, s_shpass0);
            else
                return flat_resolve<FMT, MAXM>(Q, end, ns, pN, sN, rpp, grp, w_r, s_rt, w_s, s_s, cursor, s_e, s_r0,
                                               s_m, s_pass0);
        };
        auto grab = [&]() __attribute__((always_inline)) {
            int g = 0;
            if (lane == 0) g = atomicAdd(SH ? &s_shnext : &s_next, 1);
            return min(__builtin_amdgcn_readfirstlane(g), end);
        };

        int P = P0 < 0 ? grab() : min(P0, end);
        FlatPass fc = resolve(P);
        u32x4 wa[U], wb[U];
        uint32_t sa[NSC], sb[NSC];
        load(fc.wb, fc.sb, fc.ridx, fc.srow, 0, wa, sa);
        int Pn = P < end ? grab() : end;
        FlatPass fn = resolve(Pn);
        tokens(fc);
        int ib = 0;
        // one batch: load the following one into `nx` (the next pass's first batch after the
        // last one; every field selected, so the load is unconditional), consume `cu`
        auto step = [&](u32x4 (&cu)[U], uint32_t (&cs)[NSC], u32x4 (&nx)[U],
                        uint32_t (&nsc)[NSC]) __attribute__((always_inline)) {
            const bool last = ib + 1 == nb;
            load(last ? fn.wb : fc.wb, last ? fn.sb : fc.sb, last ? fn.ridx : fc.ridx, last ? fn.srow : fc.srow,
                 last ? 0 : ib + 1, nx, nsc);
            compute(fc, ib, cu, cs);
            if (last) {
                P = Pn;
                fc = fn;
                Pn = P < end ? grab() : end;
                fn = resolve(Pn);
                tokens(fc);
                ib = 0;
            } else {
                ++ib;
            }
            return P < end;
        };
        bool more = P < end;
        while (more) {
            more = step(wa, sa, wb, sb);
            if (!more) break;
            more = step(wb, sb, wa, sa);
        }
    };
    if constexpr (ROUTE) {
        lds_wait_at_least(&s_dma, NW - T0);                // every activation row is in LDS
        run(std::true_type{}, -1, sh_end, 1);
        lds_wait_at_least(&s_tab, 1);
        run(std::false_type{}, -1, s_end, s_ns);
    } else {
        const int end = s_end;
        run(std::false_type{}, s_beg + wave, end, s_ns);
    }
    if constexpr (ROUTE) {
        // workgroup 0 writes the permutation, by the first of its waves to run out of passes
        // (written at the start, it held back every wave of workgroup 0 by that long)
        if (blockIdx.x == 0) {
            int v = 1;
            if (lane == 0) v = atomicAdd(&s_perm, 1);
            if (__builtin_amdgcn_readfirstlane(v) == 0)
                small_permutation(s_sid, T * kk, E, ra.offsets, ra.sorted, ra.p2r, lane, 64);
        }
    }
    if constexpr (STEP) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's h rows are stored
}

template <int FMT, int ACT, int MAXM, bool PAIR, bool ROUTE = false>
__global__ __launch_bounds__(kFlatThreads) void gemv_flat_kernel(const GemvParams p) {
    flat_body<FMT, ACT, MAXM, PAIR, ROUTE, false>(p, nullptr);
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
constexpr int kDcRows = 4;                 // weight rows per lane group
constexpr int kDcDepth = 2;                // batches in flight per wave
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

// Launch shape of the down-combine: fills p.G, p.nl, p.rows_per_wg and p.h_lds_bytes;
// returns the grid (row ranges, tokens), the LDS bytes and the FP8 form's batch U.
static dim3 down_combine_shape(int fmt, DownCombineParams &p, size_t *lds, int *U_out) {
    const bool mfma = fmt == kFmtMXFP4;
    const int units = fmt == kFmtMXFP4 ? p.I / 32 : p.I / 16;
    int U = 1, rpp = 4;                                    // MFMA path: 8-row tiles, the last one clamped

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
    // does not need every CU), whole passes, at most kDcMaxRows rows (kDmMaxRows on the
    // matrix cores, which keep two partial sums per row)
    const long long rows_total = (long long)p.N * p.T;
    int rpw = (int)((rows_total + 255) / 256);
    rpw = (max(rpw, rpp) + rpp - 1) / rpp * rpp;
    rpw = min(rpw, max(rpp, (mfma ? kDmMaxRows : kDcMaxRows) / rpp * rpp));
    p.rows_per_wg = rpw;
    const int nslot = p.k + (p.sw ? 1 : 0);
    p.h_lds_bytes = (int)align_up((size_t)nslot * 4 * dc_plane_ld(p.I), 1024);
    *lds = down_combine_lds(p.k, p.sw != nullptr, p.I);
    *U_out = U;
    return dim3((p.N + rpw - 1) / rpw, p.T);
}

moe_status down_combine_launch(int fmt, DownCombineParams p, hipStream_t stream) {
    const bool mfma = fmt == kFmtMXFP4;
    size_t lds = 0;
    int U = 1;
    const dim3 grid = down_combine_shape(fmt, p, &lds, &U);
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

template <int FMT, int ACT, bool PAIR, bool ROUTED>
static GemvFn pick_kernel_t(int maxm, bool wide) {
    if (wide) {
        switch (maxm) {
            case 1:
            case 2: return gemv_kernel<FMT, ACT, 2, PAIR, ROUTED, gemv_wide_threads<ACT>()>;
            case 4: return gemv_kernel<FMT, ACT, 4, PAIR, ROUTED, gemv_wide_threads<ACT>()>;
            default: return gemv_kernel<FMT, ACT, 8, PAIR, ROUTED, gemv_wide_threads<ACT>()>;
        }
    }
    switch (maxm) {
        case 1: return gemv_kernel<FMT, ACT, 1, PAIR, ROUTED, kGemvThreads>;
        case 2: return gemv_kernel<FMT, ACT, 2, PAIR, ROUTED, kGemvThreads>;
        case 4: return gemv_kernel<FMT, ACT, 4, PAIR, ROUTED, kGemvThreads>;
        default: return gemv_kernel<FMT, ACT, 8, PAIR, ROUTED, kGemvThreads>;
    }
}

template <int FMT, int ACT, bool PAIR>
static GemvFn pick_kernel_m(int maxm, bool routed, bool wide) {
    return routed ? pick_kernel_t<FMT, ACT, PAIR, true>(maxm, wide) : pick_kernel_t<FMT, ACT, PAIR, false>(maxm, wide);
}

template <int FMT, bool PAIR>
static GemvFn pick_kernel_a(int act, int maxm, bool routed, bool wide) {
    if (act == kActF32) return pick_kernel_m<FMT, kActF32, PAIR>(maxm, routed, wide);
    if (act == kActMX && FMT == kFmtMXFP4) return pick_kernel_m<kFmtMXFP4, kActMX, PAIR>(maxm, routed, wide);
    return pick_kernel_m<FMT, kActBF16, PAIR>(maxm, routed, wide);
}

static GemvFn pick_kernel(int fmt, int act, bool pair, int maxm, bool routed, bool wide) {
    if (fmt == kFmtMXFP4)
        return pair ? pick_kernel_a<kFmtMXFP4, true>(act, maxm, routed, wide)
                    : pick_kernel_a<kFmtMXFP4, false>(act, maxm, routed, wide);
    if (fmt == kFmtFP8)
        return pair ? pick_kernel_a<kFmtFP8, true>(act, maxm, routed, wide)
                    : pick_kernel_a<kFmtFP8, false>(act, maxm, routed, wide);
    return pick_kernel_a<kFmtBF16, false>(act, maxm, false, wide);
}

// LDS for staged activations per workgroup.  Small enough that several workgroups share a
// CU (occupancy matters more than the token tile: decode experts mostly own one row);
// experts with more rows than fit loop over token chunks.
constexpr size_t kGemvLdsBudget = 32 * 1024;
constexpr size_t kGemvWideLdsBudget = 96 * 1024;

template <int FMT, int ACT, bool PAIR>
static GemvFn pick_flat_m(int maxm) {
    switch (maxm) {
        case 1: return gemv_flat_kernel<FMT, ACT, 1, PAIR>;
        case 2: return gemv_flat_kernel<FMT, ACT, 2, PAIR>;
        case 4: return gemv_flat_kernel<FMT, ACT, 4, PAIR>;
        default: return gemv_flat_kernel<FMT, ACT, 8, PAIR>;
    }
}

template <int FMT, bool PAIR>
static GemvFn pick_flat_a(int act, int maxm) {
    return act == kActF32 ? pick_flat_m<FMT, kActF32, PAIR>(maxm) : pick_flat_m<FMT, kActBF16, PAIR>(maxm);
}

static GemvFn pick_flat(int fmt, int act, bool pair, int maxm) {
    if (fmt == kFmtMXFP4) return pair ? pick_flat_a<kFmtMXFP4, true>(act, maxm) : pick_flat_a<kFmtMXFP4, false>(act, maxm);
    if (fmt == kFmtFP8) return pair ? pick_flat_a<kFmtFP8, true>(act, maxm) : pick_flat_a<kFmtFP8, false>(act, maxm);
    return pick_flat_a<kFmtBF16, false>(act, maxm);
}

template <int FMT, int ACT>
static GemvFn pick_flat_route_m(int maxm) {
    switch (maxm) {
        case 1: return gemv_flat_kernel<FMT, ACT, 1, true, true>;
        case 2: return gemv_flat_kernel<FMT, ACT, 2, true, true>;
        default: return gemv_flat_kernel<FMT, ACT, 4, true, true>;
    }
}

// Workgroups of a flat launch: one per CU, or one per pass when there are fewer passes than
// CUs.  A launch of few passes (a small projection, a lone shared expert) spreads them over
// every CU: the bytes in flight scale with the CUs streaming, not with the waves of one CU.
static int flat_grid(long long passes) {
    return (int)std::min<long long>(device_cu_count(), std::max<long long>(1, passes));
}

// Shape of the routing-in-the-prologue gate/up launch: fills p.G and p.nl, the LDS bytes and
// the token tile; false when the shapes do not allow the form.
static bool gemv_route_shape(int fmt, int act, GemvParams &p, size_t *lds_out, int *maxm_out) {
    if ((fmt != kFmtMXFP4 && fmt != kFmtFP8) || act != kActBF16) return false;
    const int units = fmt == kFmtMXFP4 ? p.K / 32 : p.K / 16;
    pick_layout(units, true, &p.G, &p.nl);
    const size_t rs = align_up((size_t)p.K * 2, 1024);
    const int ng = p.route.n_group > 1 ? p.route.n_group : 1;
    const size_t lds = (size_t)p.T * rs + (ng > 1 ? (size_t)p.T * p.E * sizeof(double) : 0);
    if (p.T < 1 || p.T > 4 || p.T * p.k > 64 || p.E > 64 * kFlatTopkNK || p.n_act_rows != p.T ||
        lds > kFlatLdsBudget || (fmt == kFmtMXFP4 && units % 4 != 0) || p.G < 4)
        return false;
    int maxm = 1;
    while (maxm < p.T) maxm *= 2;
    *lds_out = lds;
    *maxm_out = maxm;
    return true;
}

bool gemv_route_launch(int fmt, int act, GemvParams p, int slots, hipStream_t stream, moe_status *st) {
    size_t lds = 0;
    int maxm = 1;
    if (!gemv_route_shape(fmt, act, p, &lds, &maxm)) return false;
    const int rpp = 32 / p.G;
    long long passes = (long long)(slots - (p.shared_slot >= 0 ? 1 : 0)) * ((p.N + rpp - 1) / rpp);
    if (p.shared_slot >= 0) passes += (p.sN + rpp - 1) / rpp;
    const int nwg = flat_grid(passes);
    GemvFn fn = fmt == kFmtMXFP4 ? pick_flat_route_m<kFmtMXFP4, kActBF16>(maxm) : pick_flat_route_m<kFmtFP8, kActBF16>(maxm);
    hipLaunchKernelGGL(fn, dim3(nwg), dim3(kFlatThreads), lds, stream, p);
    *st = launch_check("moe_route_gateup_shared: gemv_flat_kernel");
    return true;
}

moe_status gemv_launch(int fmt, int act, bool pair, GemvParams p, int slots, int max_rows_per_expert,
                       hipStream_t stream, const char *what) {
    const bool act_f32 = act == kActF32;
    const int units = fmt == kFmtMXFP4 ? p.K / 32 : (fmt == kFmtFP8 ? p.K / 16 : p.K / 8);
    pick_layout(units, pair, &p.G, &p.nl);
    const size_t row_lds = (size_t)p.K * (act_f32 ? 4 : 2);

    // Decode-sized launches (every activation row fits in LDS at once, float or bf16): the
    // flat schedule, one workgroup per CU over an equal share of the passes.
    const bool routed = p.offsets != nullptr;
    const size_t rs = align_up(row_lds, 1024);
    if (act != kActMX && p.n_act_rows >= 1 && p.n_act_rows <= kFlatMaxTok && (size_t)p.n_act_rows * rs <= kFlatLdsBudget &&
        (fmt != kFmtMXFP4 || (units % 4 == 0 && p.G >= 4)) &&
        (routed ? p.R : p.T) <= kFlatMaxSlots - 1 && (routed || p.T <= kFlatMaxTok)) {
        int want = max_rows_per_expert < 1 ? 1 : (max_rows_per_expert > 8 ? 8 : max_rows_per_expert);
        int maxm = 1;
        while (maxm < want) maxm *= 2;
        const int rpp = pair ? 32 / p.G : 64 / p.G;
        const int routed_slots = routed ? slots - (p.shared_slot >= 0 ? 1 : 0) : 1;
        long long passes = (long long)routed_slots * ((p.N + rpp - 1) / rpp);
        if (p.shared_slot >= 0) passes += (p.sN + rpp - 1) / rpp;
        const int nwg = flat_grid(passes);
        hipLaunchKernelGGL(pick_flat(fmt, act, pair, maxm), dim3(nwg), dim3(kFlatThreads), (size_t)p.n_act_rows * rs,
                           stream, p);
        return launch_check(what);
    }
    int fit = (int)(kGemvLdsBudget / row_lds);
    if (fit < 1) fit = (int)(64 * 1024 / row_lds);   // wide rows: one token per chunk
    if (fit < 1) {
        set_error("%s: an activation row of %zu bytes does not fit in LDS", what, row_lds);
        return MOE_ERR_UNSUPPORTED;
    }
    // token chunk: rows per expert that fit, at most the widest register tile (8).  When an
    // expert's rows need more than one chunk of the small budget (wide rows: two bf16 rows of
    // K = 6144 fill 24 of its 32 KiB), every further chunk streams the expert's weights
    // again; the wide form then holds up to 8 rows in 96 KiB with one workgroup (of 16 waves,
    // 8 with float32 rows) per CU, so each expert of up to 8 rows streams once.
    const int rows_needed = max_rows_per_expert < 1 ? 1 : (max_rows_per_expert > 8 ? 8 : max_rows_per_expert);
    const int fit_wide = (int)(kGemvWideLdsBudget / row_lds);
    const bool wide = rows_needed > fit && fit_wide > fit;
    const int threads = !wide ? kGemvThreads
                              : (act_f32 ? gemv_wide_threads<kActF32>() : gemv_wide_threads<kActBF16>());
    int want = rows_needed < (wide ? fit_wide : fit) ? rows_needed : (wide ? fit_wide : fit);
    want = want < 1 ? 1 : (want > 8 ? 8 : want);
    int maxm = 1;
    while (maxm < want) maxm *= 2;
    p.chunk = want;
    const int rows_per_pass = pair ? 32 / p.G : 64 / p.G;
    // aim for at most kGemvTargetWaves waves over the whole launch (rounding the rows
    // per workgroup up: a workgroup more than the target puts a fifth one on some CUs, whose
    // workgroups then finish last), at least one pass per wave; the wide form (one workgroup
    // per CU at a time) aims for 8 workgroups per CU over the launch, so the rounds balance
    const int n_grid = p.shared_slot >= 0 ? max(p.N, p.sN) : p.N;
    const long long rows_total = (long long)n_grid * slots;
    const int target_wgs = wide ? 8 * device_cu_count() : kGemvTargetWaves / (kGemvThreads / 64);
    int rpw = (int)((rows_total + target_wgs - 1) / target_wgs);
    const int min_rpw = rows_per_pass * (threads / 64);
    if (rpw < min_rpw) rpw = min_rpw;
    rpw = (rpw + rows_per_pass - 1) / rows_per_pass * rows_per_pass;
    p.rows_per_wg = rpw;
    dim3 grid((n_grid + rpw - 1) / rpw, slots);
    const size_t lds = align_up((size_t)p.chunk * row_lds, 1024);   // whole 1 KiB blocks: stage_row_dma
    GemvFn fn = pick_kernel(fmt, act, pair, maxm, p.offsets != nullptr, wide);
    hipLaunchKernelGGL(fn, grid, dim3(threads), lds, stream, p);
    return launch_check(what);
}

// ------------------------------------------------------------------ single-launch decode step
// The whole decode layer step in one launch of one workgroup per compute unit (Rulith
// Inference README, engine section: a step's routed experts in one launch, with no host
// round trip between its parts).  Three phases, separated by the flag hand-offs of
// step_sync.h:
//   1. router logits: rows b, b + nwg, ... of the router (and the shared-gate row) by
//      groups of four waves, each wave a quarter of H (router_quarter: the same sums as
//      router_logits_kernel), stored as tagged words;
//   2. top-k and gate/up (flat_body<..., ROUTE, STEP>): the shared expert's gate/up passes
//      do not depend on the routing and run while the routing waves collect every
//      workgroup's logits; then the routed passes;
//   3. down and combine (dm_body<true>): each workgroup issues its first weight loads, then
//      waits for every workgroup's h rows, over the down-combine's (row range, token) items
//      b, b + nwg, ....
// Every workgroup selects the same experts from the same logits, so each keeps its own
// routing in LDS for phase 3; workgroup 0 writes the routing results and the permutation.
template <int MAXM>
__global__ __launch_bounds__(kFlatThreads) void decode_step_kernel(const StepParams sp) {
    __shared__ StepRouting s_route;
    constexpr int NG = kFlatThreads / 64 / kRouterWaves;   // router row groups per workgroup
    __shared__ double s_rpart[NG][kRouterWaves][kRouterTB];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    const int nwg = gridDim.x;
    const uint32_t c = __builtin_amdgcn_readfirstlane(step_launch_count(sp.sync));
    StepCtx sc;
    sc.sync = sp.sync;
    sc.tag = c + 1u;
    sc.nwg = nwg;
    sc.lds = &s_route;

    // 1. router logits
    const int grp = wave / kRouterWaves, quarter = wave % kRouterWaves;
    const int nround = (sp.rows + nwg * NG - 1) / (nwg * NG);
    for (int rd = 0; rd < nround; ++rd) {
        const int row = (int)blockIdx.x + nwg * (rd * NG + grp);
        if (row < sp.rows) {
            const uint16_t *w = row < sp.E ? sp.wr + (size_t)row * sp.H : sp.wsg;
            double s[kRouterTB];
            router_quarter(sp.x, w, 0, sp.T, sp.H, quarter, s);
#pragma unroll
            for (int t = 0; t < kRouterTB; ++t) {
                if (t >= sp.T) break;
                if (lane == 0) s_rpart[grp][quarter][t] = s[t];
            }
        }
        __syncthreads();
        if (quarter == 0 && row < sp.rows && lane < sp.T) {
            const float v = router_finish(s_rpart[grp], lane);
            sp.logits[(size_t)lane * sp.rows + row] = v;
            step_put_logit(sp.sync, sc.tag, lane, row, v);
        }
        __syncthreads();
    }

    // 2. top-k, routed and shared gate/up (every wave returns with its h rows stored)
    flat_body<kFmtMXFP4, kActBF16, MAXM, true, true, true>(sp.gu, &sc);
    __syncthreads();
    if (threadIdx.x == 0) step_flag(sp.sync, sc.tag);

    // 3. down and combine
    const int nitems = sp.nx * sp.T;
    for (int v = (int)blockIdx.x; v < nitems; v += nwg) dm_body<true>(sp.dc, v % sp.nx, v / sp.nx, &sc, v == (int)blockIdx.x);
    // every workgroup has arrived at the end of phase 2 (workgroup 0 has waited for it in its
    // first item), so every one has read the launch count
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(sp.sync, c + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static bool step_fits(void (*fn)(const StepParams), int maxm, size_t lds) {
    constexpr int kMaxDev = 64, kSlots = 8;
    struct Entry { int maxm; size_t lds; bool fits; };
    static std::mutex mu;
    static Entry cache[kMaxDev][kSlots];
    static int used[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return false;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used[dev]; ++i)
        if (cache[dev][i].maxm == maxm && cache[dev][i].lds == lds) return cache[dev][i].fits;
    int per_cu = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)fn, kFlatThreads, lds);
    if (e != hipSuccess) (void)hipGetLastError();          // (a failed query only means: take the three calls)
    const bool fits = e == hipSuccess && per_cu >= 1;
    if (used[dev] < kSlots) cache[dev][used[dev]++] = Entry{maxm, lds, fits};
    return fits;
}

bool decode_step_launch(StepParams sp, hipStream_t stream, moe_status *st) {
    size_t lds_gu = 0, lds_dc = 0;
    int maxm = 1, U = 1;
    if (!gemv_route_shape(kFmtMXFP4, kActBF16, sp.gu, &lds_gu, &maxm)) return false;
    const dim3 dgrid = down_combine_shape(kFmtMXFP4, sp.dc, &lds_dc, &U);
    sp.nx = (int)dgrid.x;
    const int nwg = device_cu_count();
    if (nwg > kSyncMaxWG || sp.T > kSyncMaxT || sp.rows > kSyncRowStride || sp.H % 32 != 0 || sp.T * sp.gu.k > 64)
        return false;
    const size_t lds = std::max(lds_gu, lds_dc);
    using StepFn = void (*)(const StepParams);
    StepFn fn = maxm == 1 ? decode_step_kernel<1> : (maxm == 2 ? decode_step_kernel<2> : decode_step_kernel<4>);
    // every workgroup must be resident at once: one per CU (the occupancy query is cached per
    // device, token tile and LDS size)
    if (!step_fits(fn, maxm, lds)) return false;
    hipLaunchKernelGGL(fn, dim3(nwg), dim3(kFlatThreads), lds, stream, sp);
    *st = launch_check("moe_decode_step: decode_step_kernel");
    return true;
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

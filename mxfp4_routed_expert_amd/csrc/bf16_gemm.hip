// Prefill grouped GEMM for unquantised activations over MXFP4 expert weights.
//
// Weight-only quantisation keeps the activations as given (bf16 x, float32 h), so the
// products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) instead of the FP4 ones.
// Every weight is decoded exactly: an E2M1 code times its block's E8M0 scale is a bf16 value
// (one scaled-conversion instruction per two codes; rabbit README, architecture table, and
// the OCP MX element and scale formats).  float32 operands are split into
// hi = RN_bf16(v) and lo = RN_bf16(v - hi), two products each, together within 2^-17 |v|.
//
// Both kernels: a workgroup computes 128 rows of one expert (tokens routed to it, in sorted
// order) by a tile of output columns with 8 waves (two per SIMD), 2 along the rows x 4 along
// the columns, each owning 64 rows as 16 x 16 MFMA tiles.  The weights are the MFMA's first
// operand (rows = output columns n) and the activations its second, so a lane's four
// accumulators are four consecutive columns of one row: one 16-byte store.  The activation
// rows of a K-step, shared by all 8 waves, are staged in LDS, double-buffered: while the
// matrix cores work on step s, step s+1 (loaded into registers earlier) is written to the
// other buffer; one barrier per step.  A wave skips the MFMAs of its 16-row tiles that start
// past the expert's last row (their outputs are never stored).  The grid is persistent and walks (row tile, column
// tile) items expert by expert, in the same XCD-aware order as the FP4 grouped GEMM.
//
// gate/up (fgemm_pair_kernel): 128 columns of gate AND up at the same columns, so
// h = silu(g) * u is formed in registers.  K-steps of 64 values; the step's weight units
// (16 code bytes each) and their scales are staged in LDS next to the activations, and each
// wave decodes the 8 codes of its lane slot right before the MFMAs: LDS carries the codes,
// a quarter of the bytes of decoded bf16 weights.
// down (fgemm_down_kernel): 256 columns of one matrix, K-steps of 128 values (4 MX blocks).
// Weights never pass through LDS: for each of its four 16-column tiles a lane loads the
// 16-byte unit of row l%16, block l/16 of the step, and decodes it right before its MFMAs
// (MFMA q takes values 8q .. 8q+7 of every lane group's block); with float32 h each decoded
// weight feeds twice as many products (hi and lo), which pays for decoding it per wave.
#include <algorithm>
#include <type_traits>

#include "gemv.h"
#include "tile_sched.h"

namespace moe {

constexpr int kFPairPF = 2;               // gate/up: steps whose loads are in flight
constexpr int kFDownPF = 1;               // down: steps whose loads are in flight

constexpr int kFBM = 128;                  // rows (tokens) per tile
constexpr int kFThreads = 512;             // 8 waves: 2 along the rows x 4 along the columns

struct FGemmParams {
    const void *a;                 // activations: bf16 or float32 rows [n_arows][K]
    int gather;                    // 1: activation row = sorted_pairs[r] / k; 0: row r
    int n_arows;
    const int32_t *sorted_pairs;
    int k;
    const uint8_t *w[2];           // MXFP4 codes [E][N][K/2]
    const uint8_t *ws[2];          // E8M0 scales [E][N][K/32]
    int E, N, K;
    const int32_t *offsets;        // NULL: identity (one expert, rows 0..T-1)
    int T;
    int R;
    float *out;                    // [R][N] float32: h = silu(gate) * up, or y
};

// Item -> (expert, first row, rows of the expert, row tile, column tile).
template <bool ROUTED>
MOE_DEV void fgemm_item(const FGemmParams &p, const int *tp, int total_mt, int NT, int item, int &e, int &row0,
                        int &M, int &tile, int &nt) {
    if constexpr (ROUTED) {
        e = tile_expert(tp, p.E, item / NT);
        const int tpx = e > 0 ? tp[e - 1] : 0, te = tp[e] - tpx;
        const int r = item - NT * tpx;
        nt = r / te;
        tile = r - nt * te;
        row0 = p.offsets[e];
        M = p.offsets[e + 1] - row0;
    } else {
        e = 0;
        row0 = 0;
        M = p.T;
        nt = item / total_mt;
        tile = item - nt * total_mt;
    }
}

// Source of activation row r of a tile (rows past the expert's end repeat a valid row;
// their results are not stored).
template <bool SPLIT>
MOE_DEV const unsigned char *fgemm_arow(const FGemmParams &p, int row0, int M, int m0, int r) {
    int src = row0 + min(m0 + r, M - 1);
    if (p.gather) src = p.sorted_pairs[src] / p.k;
    src = min(max(src, 0), p.n_arows - 1);
    return (const unsigned char *)p.a + (size_t)src * p.K * (SPLIT ? 4 : 2);
}

// 8 float32 values -> bf16 hi and lo terms, 16 bytes each.  The conversions are the
// hardware's round-to-nearest-even (v_cvt_pk_bf16_f32, two values per instruction); v - hi
// is exact in float32.
MOE_DEV void split8(const u32x4 a, const u32x4 b, u32x4 &h4, u32x4 &l4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float f0 = __uint_as_float(t < 2 ? a[2 * t] : b[2 * t - 4]);
        const float f1 = __uint_as_float(t < 2 ? a[2 * t + 1] : b[2 * t - 3]);
        const bf16x2 hv = {(__bf16)f0, (__bf16)f1};
        const uint32_t hb = __builtin_bit_cast(uint32_t, hv);
        const bf16x2 lv = {(__bf16)(f0 - __uint_as_float(hb << 16)), (__bf16)(f1 - __uint_as_float(hb & 0xffff0000u))};
        h4[t] = hb;
        l4[t] = __builtin_bit_cast(uint32_t, lv);
    }
}

// ------------------------------------------------------------------ gate/up

constexpr int kPBK = 64;                   // K values per step (2 MX blocks)
constexpr int kPRow = kPBK * 2;            // LDS bytes per operand row per step (bf16)
constexpr int kPBN = 128;                  // output columns per tile and matrix

// 16-byte chunk c (of 8) of LDS row r sits at position c ^ pswz(r): an operand read (16 rows
// at one chunk) then touches 16 distinct 16-byte bank groups.
MOE_DEV int pswz(int r) { return (r >> 1) & 7; }
// Weight codes: row R's 16-byte unit u (of 2) at position u ^ ((R >> 3) & 1), so that rows
// R and R + 8 of an operand read (the same banks otherwise) use different halves.
MOE_DEV int cswz(int R, int u) { return u ^ ((R >> 3) & 1); }

template <bool SPLIT>
struct PStep {                     // one thread's loads for one K-step
    u32x4 wc;                      // 32 weight codes (one MX block)
    uint32_t wsc;                  // its scale byte
    u32x4 a[SPLIT ? 4 : 2];        // 16 activation values (bf16: 2 x 16 B; float32: 4 x 16 B)
};

template <bool SPLIT, bool ROUTED>
__global__ __launch_bounds__(kFThreads) void fgemm_pair_kernel(const FGemmParams p) {
    constexpr int PF = kFPairPF;
    constexpr int NP = SPLIT ? 2 : 1;                  // activation planes: hi (and lo)
    constexpr int kCodes = 2 * kPBN * 32;              // codes of a step: 256 weight rows x 2 units
    constexpr int kScales = 2 * kPBN * 2 * 4;          // their scales, as float32
    constexpr int kAPlane = kFBM * kPRow;              // one activation plane's step
    constexpr int kAOff = kCodes + kScales;            // activation planes after codes and scales
    constexpr int kStage = kAOff + NP * kAPlane;
    static_assert(PF >= 1 && PF <= 4, "prefetch depth");
    static_assert(2 * kPBN * 2 == kFThreads && kFBM * 4 == kFThreads, "thread roles");
    __shared__ __align__(16) unsigned char smem[2 * kStage];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kFThreads / 64];

    const int NT = (p.N + kPBN - 1) / kPBN;
    const int total_mt = ROUTED ? build_tile_prefix<kFThreads, kFBM>(p.offsets, p.E, p.R, s_tp, s_wave)
                                : (p.T + kFBM - 1) / kFBM;
    const int items = total_mt * NT;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G);
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int wm = wave >> 2, wn = wave & 3;            // 64 rows x 32 columns (per matrix)
    const int lr = lane & 15, lg = lane >> 4;          // MFMA operand row / 8-value K slot
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (p.K + kPBK - 1) / kPBK;             // K-steps (the last may hold one MX block)
    const int wmat = tid >> 8, wr = (tid >> 1) & (kPBN - 1), wb = tid & 1;   // decode: matrix, row, block
    const int ar = tid >> 2, ac = tid & 3;             // staging: row ar, values 16 ac .. 16 ac + 15

    for (int item = slot; item < items; item += G) {
        int e, row0, M, tile, nt;
        fgemm_item<ROUTED>(p, s_tp, total_mt, NT, item, e, row0, M, tile, nt);
        const int m0 = tile * kFBM, n0 = nt * kPBN;
        const size_t wrow = (size_t)e * p.N + min(n0 + wr, p.N - 1);   // rows past N: not stored
        const uint8_t *wsrc = p.w[wmat] + wrow * Kh;
        const uint8_t *ssrc = p.ws[wmat] + wrow * Kb;
        const unsigned char *asrc = fgemm_arow<SPLIT>(p, row0, M, m0, ar);

        auto issue = [&](PStep<SPLIT> &L, int s) {
            const int kb = min(2 * s + wb, Kb - 1);
            L.wc = *(const u32x4 *)(wsrc + (size_t)kb * 16);
            L.wsc = ssrc[kb];
            const int kc = min(s * kPBK + 16 * ac, p.K - 16);   // K % 32 == 0
            const u32x4 *q = (const u32x4 *)(asrc + (size_t)kc * (SPLIT ? 4 : 2));
#pragma unroll
            for (int i = 0; i < (SPLIT ? 4 : 2); ++i) L.a[i] = q[i];
        };
        auto commit = [&](const PStep<SPLIT> &L, int s, int buf) {
            unsigned char *st = smem + buf * kStage;
            const int kv = p.K - s * kPBK;                     // valid values of the step
            {
                // a unit past K: zero codes under scale 1 (the scale byte may be any value)
                const bool live = wb * 32 < kv;
                const int R = wmat * kPBN + wr;
                *(u32x4 *)(st + R * 32 + (cswz(R, wb) << 4)) = live ? L.wc : u32x4{0, 0, 0, 0};
                *(float *)(st + kCodes + (R * 2 + wb) * 4) = live ? e8m0_to_f32(L.wsc) : 1.0f;
            }
            const bool live = 16 * ac < kv;
            unsigned char *row = st + kAOff + ar * kPRow;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int off = ((2 * ac + i) ^ pswz(ar)) << 4;
                if constexpr (!SPLIT) {
                    *(u32x4 *)(row + off) = live ? L.a[i] : u32x4{0, 0, 0, 0};
                } else {
                    u32x4 h4, l4;
                    split8(L.a[2 * i], L.a[2 * i + 1], h4, l4);
                    *(u32x4 *)(row + off) = live ? h4 : u32x4{0, 0, 0, 0};
                    *(u32x4 *)(row + kAPlane + off) = live ? l4 : u32x4{0, 0, 0, 0};
                }
            }
        };

        f32x4 acc[2][2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int live_rows = M - m0;
        bool tlive[4];                                     // 16-row tiles holding a row of the expert
#pragma unroll
        for (int j = 0; j < 4; ++j) tlive[j] = __builtin_amdgcn_readfirstlane(16 * (4 * wm + j) < live_rows) != 0;

        // all: every 16-row tile of the wave holds rows (no per-tile test in the loop)
        auto compute = [&](int buf, auto all) {
            const unsigned char *st = smem + buf * kStage;
#pragma unroll
            for (int ks = 0; ks < kPBK / 32; ++ks) {
                const int c = 4 * ks + lg;
                bf16x8 bw[2][2], xa[NP][4];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        // codes 8 lg .. 8 lg + 7 of unit ks of weight row R, and its scale
                        const int R = m * kPBN + 32 * wn + 16 * i + lr;
                        const uint32_t cw = *(const uint32_t *)(st + R * 32 + (cswz(R, ks) << 4) + 4 * lg);
                        const float sc = *(const float *)(st + kCodes + (R * 2 + ks) * 4);
                        bw[m][i] = fp4x8_scaled_bf16(cw, sc);
                    }
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 64 * wm + 16 * j + lr;
                        xa[pl][j] = *(const bf16x8 *)(st + kAOff + pl * kAPlane + r * kPRow +
                                                      ((c ^ pswz(r)) << 4));
                    }
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int pl = 0; pl < NP; ++pl)
                                if (decltype(all)::value || tlive[j])
                                    acc[m][i][j] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[m][i], xa[pl][j], acc[m][i][j], 0, 0, 0);
            }
        };

        // ---- pipeline: slot s % PF holds step s's loads from their issue until commit(s),
        // one step before compute(s).  Loads and commits are unconditional (past the last
        // step they re-read clamped, valid addresses and write zeros to the buffer no wave
        // reads): a load under a branch would make the compiler drain every load at the join.
        // Only the last S % PF steps run under a guard, after the loop.
        PStep<SPLIT> L[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) issue(L[j], j);
        commit(L[0], 0, 0);
        issue(L[0], PF);
        lds_barrier();
        auto step = [&](PStep<SPLIT> &Ln, int s, auto all) {   // Ln: the slot of step s + 1
            compute(s & 1, all);
            commit(Ln, s + 1, (s + 1) & 1);
            issue(Ln, s + 1 + PF);
            lds_barrier();
        };
        const int Sf = S - S % PF;
        auto run = [&](auto all) {
            for (int s0 = 0; s0 < Sf; s0 += PF) {
#pragma unroll
                for (int j = 0; j < PF; ++j) step(L[(j + 1) % PF], s0 + j, all);
            }
#pragma unroll
            for (int j = 0; j < PF - 1; ++j)
                if (Sf + j < S) step(L[(j + 1) % PF], Sf + j, all);
        };
        // one test per item: full tiles run the loop without per-tile tests (float32 x always:
        // a second copy of its loop does not fit in the registers)
        if (SPLIT || tlive[3]) run(std::true_type{});
        else run(std::false_type{});

        // ---- epilogue: lane (lr, lg) of tile (i, j) holds columns 4 lg .. 4 lg + 3 of row lr
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int n = n0 + 32 * wn + 16 * i + 4 * lg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = m0 + 64 * wm + 16 * j + lr;
                if (r < M && n < p.N) {
                    f32x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = silu(acc[0][i][j][q]) * acc[1][i][j][q];
                    *(f32x4 *)(p.out + (size_t)(row0 + r) * p.N + n) = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ down

constexpr int kDBK = 128;                  // K values per step (4 MX blocks)
constexpr int kDRow = kDBK * 2;            // LDS bytes per activation row per step (bf16)
constexpr int kDNF = 4;                    // 16-column MFMA tiles per wave
constexpr int kDBN = 4 * 16 * kDNF;        // output columns per tile (256)

// 16-byte chunk c (of 16) of LDS row r sits at position c ^ (r & 15): an operand read (16
// rows at one chunk) touches all 16 bank groups of a 256-byte row once.
MOE_DEV int dswz(int r) { return r & 15; }

struct DActs {                     // one thread's activation loads for one K-step
    u32x4 v[8];                    // 32 float32 values
};
struct DWts {                      // one lane's weight units for one K-step
    u32x4 c[kDNF];                 // 32 codes each (one MX block)
    uint32_t s[kDNF];              // their scale bytes
};

template <bool ROUTED>
__global__ __launch_bounds__(kFThreads) void fgemm_down_kernel(const FGemmParams p) {
    constexpr int PF = kFDownPF;
    constexpr int kAPlane = kFBM * kDRow;              // one activation plane's step
    constexpr int kStage = 2 * kAPlane;                // hi and lo planes
    static_assert(PF >= 1 && PF <= 4, "prefetch depth");
    static_assert(kFBM * 4 == kFThreads, "activation staging: four threads per row");
    __shared__ __align__(16) unsigned char smem[2 * kStage];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kFThreads / 64];

    const int NT = (p.N + kDBN - 1) / kDBN;
    const int total_mt = ROUTED ? build_tile_prefix<kFThreads, kFBM>(p.offsets, p.E, p.R, s_tp, s_wave)
                                : (p.T + kFBM - 1) / kFBM;
    const int items = total_mt * NT;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G);
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int wm = wave >> 2, wn = wave & 3;            // 64 rows x 64 columns of this wave
    const int lr = lane & 15, lg = lane >> 4;          // MFMA operand row / MX block of the step
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (p.K + kDBK - 1) / kDBK;             // K-steps (the last may hold 1..4 blocks)
    const int ar = tid >> 2, ac = tid & 3;             // staging: row ar, values 32 ac .. 32 ac + 31

    for (int item = slot; item < items; item += G) {
        int e, row0, M, tile, nt;
        fgemm_item<ROUTED>(p, s_tp, total_mt, NT, item, e, row0, M, tile, nt);
        const int m0 = tile * kFBM, n0 = nt * kDBN;
        const uint8_t *wsrc[kDNF];
        const uint8_t *ssrc[kDNF];
#pragma unroll
        for (int i = 0; i < kDNF; ++i) {
            const size_t row = (size_t)e * p.N + min(n0 + 16 * (kDNF * wn + i) + lr, p.N - 1);  // past N: not stored
            wsrc[i] = p.w[0] + row * Kh;
            ssrc[i] = p.ws[0] + row * Kb;
        }
        const unsigned char *asrc = fgemm_arow<true>(p, row0, M, m0, ar);

        auto issue_w = [&](DWts &W, int s) {
            const int kb = min(4 * s + lg, Kb - 1);
#pragma unroll
            for (int i = 0; i < kDNF; ++i) {
                W.c[i] = *(const u32x4 *)(wsrc[i] + (size_t)kb * 16);
                W.s[i] = ssrc[i][kb];
            }
        };
        auto issue_a = [&](DActs &A, int s) {
            const int kc = min(s * kDBK + 32 * ac, p.K - 32);   // K % 32 == 0
            const u32x4 *q = (const u32x4 *)(asrc + (size_t)kc * 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) A.v[i] = q[i];
        };
        auto commit = [&](const DActs &A, int s, int buf) {
            unsigned char *row = smem + buf * kStage + ar * kDRow;
            const bool live = 32 * ac < p.K - s * kDBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 h4, l4;
                split8(A.v[2 * i], A.v[2 * i + 1], h4, l4);
                const int off = ((4 * ac + i) ^ dswz(ar)) << 4;
                *(u32x4 *)(row + off) = live ? h4 : u32x4{0, 0, 0, 0};
                *(u32x4 *)(row + kAPlane + off) = live ? l4 : u32x4{0, 0, 0, 0};
            }
        };

        f32x4 acc[kDNF][4];
#pragma unroll
        for (int i = 0; i < kDNF; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int live_rows = M - m0;
        bool tlive[4];                                     // 16-row tiles holding a row of the expert
#pragma unroll
        for (int j = 0; j < 4; ++j) tlive[j] = __builtin_amdgcn_readfirstlane(16 * (4 * wm + j) < live_rows) != 0;

        // all: every 16-row tile of the wave holds rows (no per-tile test in the loop)
        auto compute = [&](const DWts &W, int s, int buf, auto all) {
            const unsigned char *st = smem + buf * kStage;
            const bool wlive = 4 * s + lg < Kb;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 xa[2][4];
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 64 * wm + 16 * j + lr;
                        xa[pl][j] = *(const bf16x8 *)(st + pl * kAPlane + r * kDRow + (((4 * lg + q) ^ dswz(r)) << 4));
                    }
#pragma unroll
                for (int i = 0; i < kDNF; ++i) {
                    const uint32_t c = wlive ? W.c[i][q] : 0u;
                    const float sc = e8m0_to_f32(wlive ? W.s[i] : 127u);
                    const bf16x8 b = fp4x8_scaled_bf16(c, sc);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int pl = 0; pl < 2; ++pl)
                            if (decltype(all)::value || tlive[j])
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, xa[pl][j], acc[i][j], 0, 0, 0);
                }
            }
        };

        // ---- pipeline: weight slot s % PF holds step s's units from their issue until
        // compute(s); the activation slot holds step s + 1's rows until commit(s + 1).  Loads
        // and commits are unconditional, as in the gate/up kernel; the last S % PF steps run
        // under a guard after the loop.
        DWts WL[PF];
        DActs A;
#pragma unroll
        for (int j = 0; j < PF; ++j) issue_w(WL[j], j);
        issue_a(A, 0);
        commit(A, 0, 0);
        issue_a(A, 1);
        lds_barrier();
        auto step = [&](DWts &W, int s, auto all) {
            compute(W, s, s & 1, all);
            issue_w(W, s + PF);
            commit(A, s + 1, (s + 1) & 1);
            issue_a(A, s + 2);
            lds_barrier();
        };
        const int Sf = S - S % PF;
        auto run = [&](auto all) {
            for (int s0 = 0; s0 < Sf; s0 += PF) {
#pragma unroll
                for (int j = 0; j < PF; ++j) step(WL[j], s0 + j, all);
            }
#pragma unroll
            for (int j = 0; j < PF - 1; ++j)
                if (Sf + j < S) step(WL[j], Sf + j, all);
        };
        // one test per item: full tiles run the loop without per-tile tests
        if (tlive[3]) run(std::true_type{});
        else run(std::false_type{});

        // ---- epilogue: lane (lr, lg) of tile (i, j) holds columns 4 lg .. 4 lg + 3 of row lr
#pragma unroll
        for (int i = 0; i < kDNF; ++i) {
            const int n = n0 + 16 * (kDNF * wn + i) + 4 * lg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = m0 + 64 * wm + 16 * j + lr;
                if (r < M && n < p.N) *(f32x4 *)(p.out + (size_t)(row0 + r) * p.N + n) = acc[i][j];
            }
        }
    }
}

// ------------------------------------------------------------------ host

// The bf16 matrix-core GEMM serves unquantised activations over MXFP4 weights when there
// are enough tokens to fill 128-row tiles at least partly (prefill); decode sizes use the GEMV.
bool fgemm_wanted(const moe_expert_weights *w, int act, int T) {
    return act == MOE_ACT_FLOAT && w->format == MOE_W_MXFP4 && T >= 64 && w->d_ff % 32 == 0 &&
           w->d_model % 32 == 0;
}

// Workgroups of kernel KER resident at once on the current device (queried once per device).
template <auto KER>
static int fgemm_resident() {
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KER, kFThreads, 0) != hipSuccess || per_cu <= 0)
            per_cu = 1;
        cache[dev] = cus * per_cu;
    }
    return cache[dev];
}

// Persistent launch: at most one wave of resident workgroups.  The row tiles are bounded by
// (experts with rows) + R / 128 >= sum over experts of ceil(M_e / 128).
template <auto KER, bool ROUTED>
static moe_status fgemm_run(const FGemmParams &p, int BN, hipStream_t stream, const char *what) {
    const int64_t mt_bound = ROUTED ? (int64_t)std::min(p.E, p.R) + p.R / kFBM : (p.T + kFBM - 1) / kFBM;
    const int64_t items = mt_bound * ((p.N + BN - 1) / BN);
    const int64_t g = std::min<int64_t>(items, fgemm_resident<KER>());
    if (g <= 0) return MOE_OK;
    hipLaunchKernelGGL(KER, dim3((unsigned)g), dim3(kFThreads), 0, stream, p);
    return launch_check(what);
}

moe_status fgemm_gateup_launch(const moe_expert_weights *w, int T, int k, const void *x, bool x_f32,
                               const int32_t *offsets, const int32_t *sorted_pairs, int R, float *h,
                               hipStream_t stream) {
    FGemmParams p = {};
    p.a = x;
    p.gather = offsets ? 1 : 0;
    p.n_arows = T;
    p.sorted_pairs = sorted_pairs;
    p.k = k > 0 ? k : 1;
    p.w[0] = w->gate;
    p.w[1] = w->up;
    p.ws[0] = (const uint8_t *)w->gate_s;
    p.ws[1] = (const uint8_t *)w->up_s;
    p.E = w->num_experts;
    p.N = w->d_ff;
    p.K = w->d_model;
    p.offsets = offsets;
    p.T = T;
    p.R = R;
    p.out = h;
    const char *what = "moe_expert_gateup (bf16 GEMM)";
    if (offsets)
        return x_f32 ? fgemm_run<fgemm_pair_kernel<true, true>, true>(p, kPBN, stream, what)
                     : fgemm_run<fgemm_pair_kernel<false, true>, true>(p, kPBN, stream, what);
    return x_f32 ? fgemm_run<fgemm_pair_kernel<true, false>, false>(p, kPBN, stream, what)
                 : fgemm_run<fgemm_pair_kernel<false, false>, false>(p, kPBN, stream, what);
}

moe_status fgemm_down_launch(const moe_expert_weights *w, const float *h, const int32_t *offsets, int R, float *y,
                             hipStream_t stream) {
    FGemmParams p = {};
    p.a = h;
    p.gather = 0;
    p.n_arows = R;
    p.k = 1;
    p.w[0] = w->down;
    p.ws[0] = (const uint8_t *)w->down_s;
    p.E = w->num_experts;
    p.N = w->d_model;
    p.K = w->d_ff;
    p.offsets = offsets;
    p.T = R;
    p.R = R;
    p.out = y;
    const char *what = "moe_expert_down (bf16 GEMM)";
    return offsets ? fgemm_run<fgemm_down_kernel<true>, true>(p, kDBN, stream, what)
                   : fgemm_run<fgemm_down_kernel<false>, false>(p, kDBN, stream, what);
}

}  // namespace moe

// Prefill grouped GEMM for unquantised activations over MXFP4 expert weights.
//
// Weight-only quantisation keeps the activations as given (bf16 x, float32 h), so the
// products run on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) instead of the FP4 ones.
// Every weight is decoded exactly: an E2M1 code times its block's E8M0 scale is a bf16 value
// (one scaled-conversion instruction per two codes; rabbit README, architecture table, and
// the OCP MX element and scale formats).  float32 operands are split into
// hi = RN_bf16(v) and lo = RN_bf16(v - hi), two products each, together within 2^-17 |v|.
//
// Tile: a workgroup computes 128 rows of one expert (tokens routed to it, in sorted order)
// by 128 output columns -- of gate AND up for the SwiGLU pair, at the same columns, so
// h = silu(g) * u is formed in registers.  Its 8 waves (two per SIMD) each own 64 rows x
// 32 columns per matrix as 4 x 2 MFMA tiles of 16 x 16.  The weights are the MFMA's first
// operand (rows = output columns n) and the activations its second, so a lane's four
// accumulators are four consecutive columns of one row: one 16-byte store.
// K advances in steps of 64 values.  A step's weight codes and scales and its activation
// rows are loaded into registers MOE_FGEMM_PF steps ahead; when a step's turn comes its
// codes are decoded to bf16 and written with the activation rows into one of two LDS
// buffers while the matrix cores work on the other, one barrier per step.
// The grid is persistent and walks (row tile, column tile) items expert by expert, with
// the same XCD-aware order as the FP4 grouped GEMM.
#include <algorithm>

#include "gemv.h"
#include "tile_sched.h"

namespace moe {

constexpr int kFBM = 128;                  // rows (tokens) per tile
constexpr int kFBN = 128;                  // output columns per tile and matrix
constexpr int kFBK = 64;                   // K values per step
constexpr int kFThreads = 512;             // 8 waves: 2 along the rows x 4 along the columns
constexpr int kFRow = kFBK * 2;            // LDS bytes per operand row per step (bf16)
#ifndef MOE_USE_BF16_GEMM
#define MOE_USE_BF16_GEMM 1                // 0: prefill with unquantised activations on the GEMV
#endif
#ifndef MOE_FGEMM_PF
#define MOE_FGEMM_PF 3                     // steps whose loads are in flight
#endif
constexpr int kFPf = MOE_FGEMM_PF;
static_assert(kFPf >= 1 && kFPf <= 4, "prefetch depth");

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

// 16-byte chunk c (8 values) of LDS row r sits at chunk position c ^ fswz(r): an operand read
// (16 rows at one chunk) then touches 16 distinct 16-byte bank groups.
MOE_DEV int fswz(int r) { return (r >> 1) & 7; }

template <bool SPLIT>
struct FStep {                     // one thread's loads for one K-step
    u32x4 wc;                      // 32 weight codes (one MX block)
    uint32_t wsc;                  // its scale byte
    u32x4 a[SPLIT ? 4 : 2];        // 16 activation values (bf16: 2 x 16 B; float32: 4 x 16 B)
};

template <bool PAIR, bool SPLIT, bool ROUTED>
__global__ __launch_bounds__(kFThreads) void fgemm_kernel(const FGemmParams p) {
    constexpr int NM = PAIR ? 2 : 1;
    constexpr int NP = SPLIT ? 2 : 1;                  // activation planes: hi (and lo)
    constexpr int kWPlane = kFBN * kFRow;              // one matrix's decoded step
    constexpr int kAPlane = kFBM * kFRow;              // one activation plane's step
    constexpr int kStage = NM * kWPlane + NP * kAPlane;
    constexpr int kWTasks = NM * kFBN * 2;             // (matrix, row, MX block) per step
    static_assert(kWTasks % 64 == 0 && kWTasks <= kFThreads && kFBM * 4 == kFThreads, "thread roles");
    __shared__ __align__(16) unsigned char smem[2 * kStage];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kFThreads / 64];

    const int NT = (p.N + kFBN - 1) / kFBN;
    const int total_mt = ROUTED ? build_tile_prefix<kFThreads, kFBM>(p.offsets, p.E, p.R, s_tp, s_wave)
                                : (p.T + kFBM - 1) / kFBM;
    const int items = total_mt * NT;
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G);
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int wm = wave >> 2, wn = wave & 3;            // 64-row x 32-column block of this wave
    const int lr = lane & 15, lg = lane >> 4;          // MFMA operand row / 8-value K slot
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (p.K + kFBK - 1) / kFBK;             // K-steps (the last may hold one MX block)
    // weight-decode role: matrix wm_, row wr, MX block wb of the step
    const bool wrole = tid < kWTasks;
    const int wm_ = tid / (2 * kFBN), wr = (tid >> 1) & (kFBN - 1), wb = tid & 1;
    // activation role: row ar, values 16 * ac .. 16 * ac + 15 of the step
    const int ar = tid >> 2, ac = tid & 3;

    for (int item = slot; item < items; item += G) {
        int e = 0, tile = 0, nt = 0, row0 = 0, M = p.T;
        if constexpr (ROUTED) {
            e = tile_expert(s_tp, p.E, item / NT);
            const int tpx = e > 0 ? s_tp[e - 1] : 0, te = s_tp[e] - tpx;
            const int r = item - NT * tpx;
            nt = r / te;
            tile = r - nt * te;
            row0 = p.offsets[e];
            M = p.offsets[e + 1] - row0;
        } else {
            nt = item / total_mt;
            tile = item - nt * total_mt;
        }
        const int m0 = tile * kFBM, n0 = nt * kFBN;

        // this thread's source rows (rows past the expert's or the matrix's end repeat a
        // valid row; their results are not stored)
        const size_t wrow = ((size_t)e * p.N + min(n0 + wr, p.N - 1));
        const uint8_t *wsrc = p.w[PAIR ? wm_ : 0] + wrow * Kh;
        const uint8_t *ssrc = p.ws[PAIR ? wm_ : 0] + wrow * Kb;
        int src = row0 + min(m0 + ar, M - 1);
        if (p.gather) src = p.sorted_pairs[src] / p.k;
        src = min(max(src, 0), p.n_arows - 1);
        const unsigned char *asrc =
            (const unsigned char *)p.a + (size_t)src * p.K * (SPLIT ? 4 : 2);

        auto issue = [&](FStep<SPLIT> &L, int s) {
            if (wrole) {
                const int kb = min(2 * s + wb, Kb - 1);
                L.wc = *(const u32x4 *)(wsrc + (size_t)kb * 16);
                L.wsc = ssrc[kb];
            }
            const int kc = min(s * kFBK + 16 * ac, p.K - 16);   // K % 32 == 0
            const u32x4 *q = (const u32x4 *)(asrc + (size_t)kc * (SPLIT ? 4 : 2));
#pragma unroll
            for (int i = 0; i < (SPLIT ? 4 : 2); ++i) L.a[i] = q[i];
        };
        auto commit = [&](const FStep<SPLIT> &L, int s, int buf) {
            unsigned char *st = smem + buf * kStage;
            const int kv = p.K - s * kFBK;                     // valid values of the step
            if (wrole) {
                bf16x8 v[4];
                unit_to_bf16x8(L.wc, e8m0_to_f32(L.wsc), v);
                const bool live = wb * 32 < kv;
                unsigned char *row = st + wm_ * kWPlane + wr * kFRow;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(u32x4 *)(row + (((4 * wb + q) ^ fswz(wr)) << 4)) =
                        live ? __builtin_bit_cast(u32x4, v[q]) : u32x4{0, 0, 0, 0};
            }
            const bool live = 16 * ac < kv;
            unsigned char *row = st + NM * kWPlane + ar * kFRow;
            if constexpr (!SPLIT) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    *(u32x4 *)(row + (((2 * ac + i) ^ fswz(ar)) << 4)) = live ? L.a[i] : u32x4{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    uint32_t hb[8], lb[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float f = __uint_as_float(L.a[2 * i + t / 4][t % 4]);
                        hb[t] = bf16_rne_bits(f);
                        lb[t] = bf16_rne_bits(f - __uint_as_float(hb[t] << 16));
                    }
                    const u32x4 h4 = {hb[0] | hb[1] << 16, hb[2] | hb[3] << 16, hb[4] | hb[5] << 16,
                                      hb[6] | hb[7] << 16};
                    const u32x4 l4 = {lb[0] | lb[1] << 16, lb[2] | lb[3] << 16, lb[4] | lb[5] << 16,
                                      lb[6] | lb[7] << 16};
                    const int off = ((2 * ac + i) ^ fswz(ar)) << 4;
                    *(u32x4 *)(row + off) = live ? h4 : u32x4{0, 0, 0, 0};
                    *(u32x4 *)(row + kAPlane + off) = live ? l4 : u32x4{0, 0, 0, 0};
                }
            }
        };

        f32x4 acc[NM][2][4];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](int buf) {
            const unsigned char *st = smem + buf * kStage;
#pragma unroll
            for (int ks = 0; ks < kFBK / 32; ++ks) {
                const int c = 4 * ks + lg;
                bf16x8 bw[NM][2], xa[NP][4];
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int r = 32 * wn + 16 * i + lr;
                        bw[m][i] = *(const bf16x8 *)(st + m * kWPlane + r * kFRow + ((c ^ fswz(r)) << 4));
                    }
#pragma unroll
                for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 64 * wm + 16 * j + lr;
                        xa[pl][j] = *(const bf16x8 *)(st + NM * kWPlane + pl * kAPlane + r * kFRow +
                                                      ((c ^ fswz(r)) << 4));
                    }
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int pl = 0; pl < NP; ++pl)
                                acc[m][i][j] =
                                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[m][i], xa[pl][j], acc[m][i][j], 0, 0, 0);
            }
        };

        // ---- pipeline: slot s % PF holds step s's loads from its issue until its commit
        FStep<SPLIT> L[kFPf];
#pragma unroll
        for (int j = 0; j < kFPf; ++j)
            if (j < S) issue(L[j], j);
        commit(L[0], 0, 0);
        if (kFPf < S) issue(L[0], kFPf);
        lds_barrier();
        for (int s0 = 0; s0 < S; s0 += kFPf) {
#pragma unroll
            for (int j = 0; j < kFPf; ++j) {
                const int s = s0 + j;
                if (s < S) {
                    compute(s & 1);
                    const int sn = s + 1;
                    if (sn < S) {
                        commit(L[(j + 1) % kFPf], sn, sn & 1);
                        if (sn + kFPf < S) issue(L[(j + 1) % kFPf], sn + kFPf);
                    }
                    lds_barrier();
                }
            }
        }

        // ---- epilogue: lane (lr, lg) of tile (i, j) holds columns 4 lg .. 4 lg + 3 of row lr
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int n = n0 + 32 * wn + 16 * i + 4 * lg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = m0 + 64 * wm + 16 * j + lr;
                if (r < M && n < p.N) {
                    f32x4 v;
                    if constexpr (PAIR) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = silu(acc[0][i][j][q]) * acc[1][i][j][q];
                    } else {
                        v = acc[0][i][j];
                    }
                    *(f32x4 *)(p.out + (size_t)(row0 + r) * p.N + n) = v;
                }
            }
        }
    }
}

// The bf16 matrix-core GEMM serves unquantised activations over MXFP4 weights when there
// are enough tokens to fill 128-row tiles at least partly (prefill); decode sizes use the GEMV.
bool fgemm_wanted(const moe_expert_weights *w, int act, int T) {
    return MOE_USE_BF16_GEMM && act == MOE_ACT_FLOAT && w->format == MOE_W_MXFP4 && T >= 64 && w->d_ff % 32 == 0 &&
           w->d_model % 32 == 0;
}

template <bool PAIR, bool SPLIT, bool ROUTED>
static int fgemm_resident() {
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fgemm_kernel<PAIR, SPLIT, ROUTED>, kFThreads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cache[dev] = cus * per_cu;
    }
    return cache[dev];
}

// Persistent launch: at most one wave of resident workgroups.  `mt_bound` bounds the row
// tiles (sum over experts of ceil(M_e / 128) <= experts with rows + R / 128).
template <bool PAIR, bool SPLIT, bool ROUTED>
static moe_status fgemm_run(const FGemmParams &p, hipStream_t stream, const char *what) {
    const int64_t mt_bound = ROUTED ? (int64_t)std::min(p.E, p.R) + p.R / kFBM : (p.T + kFBM - 1) / kFBM;
    const int64_t items = mt_bound * ((p.N + kFBN - 1) / kFBN);
    const int64_t g = std::min<int64_t>(items, fgemm_resident<PAIR, SPLIT, ROUTED>());
    if (g <= 0) return MOE_OK;
    hipLaunchKernelGGL((fgemm_kernel<PAIR, SPLIT, ROUTED>), dim3((unsigned)g), dim3(kFThreads), 0, stream, p);
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
        return x_f32 ? fgemm_run<true, true, true>(p, stream, what) : fgemm_run<true, false, true>(p, stream, what);
    return x_f32 ? fgemm_run<true, true, false>(p, stream, what) : fgemm_run<true, false, false>(p, stream, what);
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
    return offsets ? fgemm_run<false, true, true>(p, stream, what) : fgemm_run<false, true, false>(p, stream, what);
}

}  // namespace moe

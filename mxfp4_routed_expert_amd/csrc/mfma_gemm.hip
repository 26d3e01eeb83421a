// Prefill grouped GEMM on the gfx950 block-scaled FP4 matrix instructions.
//
// With MX-quantised activations both operands of every expert product are MXFP4: 32-value
// E2M1 blocks sharing one E8M0 scale (the format the pages name: rabbit README, opening
// section and architecture table).  v_mfma_scale_f32_32x32x64_f8f6f4 takes exactly that:
// lane l supplies 16 bytes (one 32-value block) of row l%32, K-block l/32, and the block's
// scale byte; it accumulates the scaled products in float32.
//
// Tile: a workgroup computes 128 rows of one expert (tokens routed to it, in sorted order)
// by 128 output columns -- of gate AND up for the SwiGLU pair.  Its 8 waves (two per SIMD,
// so one wave's matrix work covers the other's barrier and LDS waits) each own 64 rows x 32
// columns as 2 x 1 MFMA tiles per matrix.  K advances in steps of 256 values; a
// step's A rows (gathered token rows), B rows (weight rows) and scale windows travel from
// global memory straight into LDS (global_load_lds), a whole 128-byte line per row, while
// the matrix cores work on the previous step.
// Epilogue, gate/up: h = silu(g) * u, staged through LDS so that each lane owns a row's
// 32-column block and OCP-MX quantises it alone (block maximum, 16 packed code bytes, one
// scale byte).  Epilogue, down: float32 rows of y.
// The grid is persistent (one wave of resident workgroups); each workgroup turns
// expert_offsets into a prefix of row tiles per expert in LDS and walks its share of the
// (row tile, column tile) items, so no workgroup is launched for tiles that do not exist.
#include <algorithm>
#include <type_traits>

#include "gemv.h"
#include "tile_sched.h"

namespace moe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kGBM = 128;          // rows (tokens) per workgroup tile
constexpr int kGBN = 128;          // output columns per workgroup tile
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8           // waves per workgroup: 4 (one per SIMD) or 8 (two per SIMD)
#endif
constexpr int kNW = MOE_GEMM_WAVES;
constexpr int kGThreads = 64 * kNW;
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN (MOE_GEMM_WAVES == 8 ? 4 : 2)   // waves along the output columns
#endif
constexpr int kWN = MOE_GEMM_WN;
constexpr int kWM = kNW / kWN;                 // waves along the rows
constexpr int kTM = kGBM / 32 / kWM;           // 32-row MFMA tiles per wave
constexpr int kTN = kGBN / 32 / kWN;           // 32-column MFMA tiles per wave and matrix
static_assert((kNW == 4 || kNW == 8) && kTM >= 1 && kTN >= 1 && 32 * kTM * kTN % 64 == 0, "wave layout");

struct GemmParams {
    const uint8_t *a;              // A codes: token rows [n_arows][K/2] (gather) or rows [R][K/2]
    const uint8_t *as;             // A scales [..][K/32]
    int gather;                    // 1: A row = sorted_pairs[r] / k
    int n_arows;
    const int32_t *sorted_pairs;
    int k;
    const uint8_t *w[2];           // weight codes [E][N][K/2]
    const uint8_t *ws[2];          // weight scales [E][N][K/32]
    int E, N, K;
    const int32_t *offsets;        // NULL: identity (one expert, rows 0..T-1)
    int T;
    int R;
    float *out;                    // [R][N] float32 (h before quantisation for gate/up; y for down)
    uint8_t *oq;                   // gate/up: h codes [R][N/2]
    uint8_t *os;                   // gate/up: h scales [R][N/32]
};

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about 2 ulp).
MOE_DEV float silu_fast(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}

MOE_DEV uint32_t e2m1_code_of(float a) {   // same midpoint rule as the activation quantiser
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
           (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}


// Asynchronous global -> LDS copy (global_load_lds): lane l reads base + voff (+ OFF) and
// its bytes land at dst + l * size (base and dst are the same in every lane; the
// instruction takes dst from M0).  Written as asm so that the compiler does not add a
// wait for all copies in flight before every LDS read; the pipeline below waits for
// exactly the copies it needs.  The instruction has no register result, so nothing the
// compiler allocates is written when it completes.
template <int OFF>
MOE_DEV void dma16(const uint8_t *base, uint32_t voff, const unsigned char *dst) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(base), "i"(OFF), "{m0}"(l) : "memory");
}
MOE_DEV void dma4(const uint8_t *base, uint32_t voff, const unsigned char *dst) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(l) : "memory");
}
MOE_DEV const uint8_t *uniform_ptr(const void *q) {
    const uint64_t v = (uint64_t)(uintptr_t)q;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Wait until at most N of this wave's memory operations are outstanding, finish its LDS
// reads, then meet the other waves.  One asm block, so no memory access moves across it.
template <int N>
MOE_DEV void wait_vm_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

// K-step of MOE_GEMM_KSTEP values (256: each operand row contributes one whole 128-byte
// line per step; 128: half a line, so that more steps fit in LDS at once).
#ifndef MOE_GEMM_KSTEP
#define MOE_GEMM_KSTEP 256
#endif
constexpr int kGStep = MOE_GEMM_KSTEP;
constexpr int kRowB = kGStep / 2;              // code bytes per row per step
constexpr int kCh = kRowB / 16;                // 16-byte chunks (K-blocks) per row per step
constexpr int kRpc = 1024 / kRowB;             // rows moved by one 1-KB copy
constexpr int kRowsPW = kGBM / kNW;            // rows of each operand a wave copies
constexpr int kCpo = kRowsPW / kRpc;           // copies per operand per wave
constexpr int kScB = 16;                       // LDS bytes per scale row per step (window)
static_assert(kGStep == 256 || kGStep == 128, "K-step");

// Chunk position of chunk c of row r in LDS: rows sharing a 256-byte bank period get
// different chunk keys, so an operand read (16 rows at one chunk) hits 16 bank groups.
MOE_DEV int chunk_swz(int r) { return (r / (256 / kRowB)) & (kCh - 1); }

template <bool PAIR>
constexpr int gemm_stages() { return kGStep == 256 ? (PAIR ? 2 : 3) : (PAIR ? 5 : 7); }   // steps resident in LDS

template <bool PAIR, bool ROUTED>
__global__ __launch_bounds__(kGThreads) void mxgemm_kernel(const GemmParams p) {
    constexpr int NM = PAIR ? 2 : 1;
    constexpr int kStages = gemm_stages<PAIR>();
    constexpr int kA = kGBM * kRowB;                   // A codes of a step
    constexpr int kB = NM * kGBN * kRowB;              // B codes of a step
    constexpr int kSRows = kGBM + NM * kGBN;           // scale rows: A, then each matrix's
    constexpr int kStage = kA + kB + kSRows * kScB;
    constexpr int kCodeCopies = (kGBM + NM * kGBN) / kRpc / kNW;   // 1-KB copies per wave
    constexpr int kScCopies = kSRows / 16 / kNW;       // scale copies (16 rows x 4 dwords) per wave
    constexpr int kOps = kCodeCopies + kScCopies;      // memory operations per wave per stage
    static_assert(kSRows % (16 * kNW) == 0 && kRowsPW % kRpc == 0, "copy split");
    static_assert((kStages - 2) * kOps <= 63, "vmcnt limit");
    __shared__ __align__(16) unsigned char smem[kStages * kStage];
    __shared__ uint8_t s_off[kSRows];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kGThreads / 64];

    const int NT = (p.N + kGBN - 1) / kGBN;
    const int total_mt = ROUTED ? build_tile_prefix<kGThreads, kGBM>(p.offsets, p.E, p.R, s_tp, s_wave) : (p.T + kGBM - 1) / kGBM;
    const int items = total_mt * NT;
    // Items are ordered expert by expert, then by column tile, then by row tile, and each
    // round of G workgroups hands XCD x (workgroups x, x+8, ...) a contiguous run of G/8
    // items: the row tiles of one expert that share a column tile of weights run at the
    // same time on the same XCD, so those weight bytes come from that XCD's L2.
    const int G = gridDim.x;
    const int slot = xcd_slot(blockIdx.x, G);
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave / kWN, wn = wave % kWN;        // output block of this wave
    const int hr = lane & 31, hb = lane >> 5;          // MFMA operand row / K-block of this lane
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (Kb + kCh - 1) / kCh;                // K-steps

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
        const int m0 = tile * kGBM;
        const int n0 = nt * kGBN;

        // Source row of A row r of the tile (rows past the expert's end repeat a valid row).
        auto a_src_row = [&](int r) {
            int src = row0 + min(m0 + r, M - 1);
            if (p.gather) src = p.sorted_pairs[src] / p.k;
            return min(max(src, 0), p.n_arows - 1);
        };
        auto b_src_row = [&](int n) { return min(n0 + n, p.N - 1); };

        // ---- copies.  A step's codes sit row-major in LDS, kRowB bytes per row, with the
        // 16-byte chunk c of row r stored at chunk position c ^ chunk_swz(r): one 1-KB copy
        // moves kRpc rows, kCh lanes per row, and an MFMA operand read (rows r .. r+15 at one
        // chunk, served 16 lanes per LDS cycle) hits 16 distinct 16-byte bank groups.  Wave w
        // copies rows kRowsPW*w .. kRowsPW*(w+1)-1 of A and of each B matrix.
        const int eu = __builtin_amdgcn_readfirstlane(e);
        const uint8_t *a_base = uniform_ptr(p.a);
        const uint8_t *b_base[NM], *bs_base[NM];
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
            b_base[mi] = uniform_ptr(p.w[mi] + (size_t)eu * p.N * Kh);
            bs_base[mi] = uniform_ptr(p.ws[mi] + (size_t)eu * p.N * Kb);
        }
        const int cr = lane / kCh;                         // copy lane: row within the copy
        uint32_t a_off[kCpo], b_off[kCpo];
#pragma unroll
        for (int t = 0; t < kCpo; ++t) {
            a_off[t] = (uint32_t)a_src_row(kRowsPW * wave + kRpc * t + cr) * Kh;
            b_off[t] = (uint32_t)b_src_row(kRowsPW * wave + kRpc * t + cr) * Kh;
        }
        // Scale rows: 4 lanes per row, dword d of the row's window starting at the aligned
        // dword that holds the step's first byte.  A dword is fetched only when it holds a
        // byte of the step (otherwise the window's first dword is fetched again), so every
        // fetched dword lies inside the array.
        const int sd = lane & 3;
        const uint8_t *sc_base[kScCopies];
        uint32_t sc_off[kScCopies];
#pragma unroll
        for (int i = 0; i < kScCopies; ++i) {
            const int q0 = __builtin_amdgcn_readfirstlane(16 * (kScCopies * wave + i));   // first row of the copy
            const int q = q0 + (lane >> 2);
            sc_base[i] = q0 < kGBM ? uniform_ptr(p.as) : bs_base[q0 < kGBM + kGBN ? 0 : NM - 1];
            sc_off[i] = q < kGBM ? (uint32_t)a_src_row(q) * Kb : (uint32_t)b_src_row((q - kGBM) & (kGBN - 1)) * Kb;
            if (sd == 0) s_off[q] = (uint8_t)((uintptr_t)(sc_base[i] + sc_off[i]) & 3u);
        }
        __syncthreads();
        uint32_t sc_mis[kScCopies];
#pragma unroll
        for (int i = 0; i < kScCopies; ++i) sc_mis[i] = s_off[16 * (kScCopies * wave + i) + (lane >> 2)];
        // Consumer side: LDS byte (step-relative) of block 0 of each scale row this lane feeds.
        int sa_at[kTM], sb_at[NM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int r = 32 * (kTM * wm + i) + hr;
            sa_at[i] = kA + kB + r * kScB + s_off[r] + hb;
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int mi = 0; mi < NM; ++mi) {
                const int q = kGBM + mi * kGBN + 32 * (kTN * wn + j) + hr;
                sb_at[mi][j] = kA + kB + q * kScB + s_off[q] + hb;
            }

        // Issue the copies of step s into its stage buffer.  Steps past the end re-fetch the
        // last step (never read); K-blocks past the end of a row are clamped to its last one.
        auto issue = [&](int s) {
            const int sc = min(s, S - 1);
            unsigned char *st = smem + (s % kStages) * kStage;
#pragma unroll
            for (int t = 0; t < kCpo; ++t) {
                const int cc = (lane % kCh) ^ chunk_swz(kRowsPW * wave + kRpc * t + cr);   // chunk this lane fetches
                const uint32_t ko = (uint32_t)min(kCh * sc + cc, Kb - 1) * 16;
                dma16<0>(a_base, a_off[t] + ko, st + (kRowsPW * wave + kRpc * t) * kRowB);
#pragma unroll
                for (int mi = 0; mi < NM; ++mi)
                    dma16<0>(b_base[mi], b_off[t] + ko, st + kA + (mi * kGBN + kRowsPW * wave + kRpc * t) * kRowB);
            }
            const int last = min(kCh, Kb - kCh * sc) - 1;  // last block of the step in the row
#pragma unroll
            for (int i = 0; i < kScCopies; ++i) {
                const uint32_t o = sc_mis[i];
                const uint32_t need = (o + (uint32_t)last) >> 2;   // dwords 0..need hold bytes of the step
                const uint32_t v = sc_off[i] + (uint32_t)kCh * sc - o + ((uint32_t)sd <= need ? 4u * sd : 0u);
                dma4(sc_base[i], v, st + kA + kB + (16 * (kScCopies * wave + i)) * kScB);
            }
        };

        // Operands of one 64-value K-quarter q of a step: chunk 2q + hb of each row.
        struct Quarter {
            u32x4 a[kTM], b[NM][kTN];
            int sa[kTM], sb[NM][kTN];
        };
        auto read = [&](const unsigned char *st, int q, Quarter &f) {
            const int c = 2 * q + hb;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int r = 32 * (kTM * wm + i) + hr;
                f.a[i] = *(const u32x4 *)(st + r * kRowB + ((c ^ chunk_swz(r)) << 4));
                f.sa[i] = st[sa_at[i] + 2 * q];
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int mi = 0; mi < NM; ++mi) {
                    const int n = mi * kGBN + 32 * (kTN * wn + j) + hr;
                    f.b[mi][j] = *(const u32x4 *)(st + kA + n * kRowB + ((c ^ chunk_swz(n)) << 4));
                    f.sb[mi][j] = st[sb_at[mi][j] + 2 * q];
                }
        };
        // K-blocks past the end of K (last step only): zero A codes, unit scales.
        auto kill = [&](int s, int q, Quarter &f) {
            if (kCh * s + 2 * q + hb < Kb) return;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                f.a[i] = u32x4{0, 0, 0, 0};
                f.sa[i] = 127;
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int mi = 0; mi < NM; ++mi) f.sb[mi][j] = 127;
        };

        f32x16 acc[NM][kTM][kTN];
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mi][i][j][v] = 0.0f;
        // 32-row MFMA tiles of this wave that hold no row of the expert are skipped: their
        // outputs are never stored.  An expert with at most 64 rows in a tile (most of them
        // under skewed routing) then costs half the matrix work; the waves of rows 0-63 and
        // 64-127 share each SIMD, so the remaining work stays spread over all four.
        bool tlive[kTM];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
            tlive[i] = __builtin_amdgcn_readfirstlane(32 * (kTM * wm + i) < M - m0 ? 1 : 0) != 0;
        auto mma = [&](const Quarter &f) {
#pragma unroll
            for (int mi = 0; mi < NM; ++mi)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int i = 0; i < kTM; ++i) {
                        if (!tlive[i]) continue;
                        const u32x4 av = f.a[i], bv = f.b[mi][j];
                        acc[mi][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            i32x8_t{(int)av[0], (int)av[1], (int)av[2], (int)av[3], 0, 0, 0, 0},
                            i32x8_t{(int)bv[0], (int)bv[1], (int)bv[2], (int)bv[3], 0, 0, 0, 0}, acc[mi][i][j], 4, 4,
                            0, f.sa[i], 0, f.sb[mi][j]);
                    }
        };

        // Pipeline: kStages steps in LDS.  At step s, stage s must have landed (the later
        // kStages-2 may still be in flight); the barrier also tells every wave that step s-1's
        // buffer has been read, so step s+kStages-1 can refill it.  Within a step the next
        // quarter's operands load while the current quarter's MFMAs run.
        auto step = [&](int s, auto last) {
            wait_vm_and_barrier<(kStages - 2) * kOps>();
            issue(s + kStages - 1);
            const unsigned char *st = smem + (s % kStages) * kStage;
            Quarter f0, f1;
            read(st, 0, f0);
#pragma unroll
            for (int q = 0; q < kCh / 2; q += 2) {
                read(st, q + 1, f1);
                if constexpr (decltype(last)::value) kill(s, q, f0);
                mma(f0);
                if (q + 2 < kCh / 2) read(st, q + 2, f0);
                if constexpr (decltype(last)::value) kill(s, q + 1, f1);
                mma(f1);
            }
        };
#pragma unroll
        for (int s = 0; s < kStages - 1; ++s) issue(s);
        for (int s = 0; s < S - 1; ++s) step(s, std::false_type{});
        step(S - 1, std::true_type{});
        wait_vm_and_barrier<0>();                          // no copy in flight past this point

        // ---- epilogue.  Lane l holds C[8(v/4) + 4(l/32) + v%4][l%32] of each 32x32 tile.
        if constexpr (!PAIR) {
            // y rows: each (tile, v) is 32 consecutive float32 columns of one row per half-wave
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = m0 + 32 * (kTM * wm + i) + 8 * (v >> 2) + 4 * hb + (v & 3);
                    if (r >= M) continue;
                    const size_t orow = (size_t)(row0 + r);
#pragma unroll
                    for (int j = 0; j < kTN; ++j) {
                        const int n = n0 + 32 * (kTN * wn + j) + hr;
                        if (n < p.N) p.out[orow * p.N + n] = acc[0][i][j][v];
                    }
                }
        } else {
            // h = silu(g) * u goes through LDS (the stage buffers are idle now): the wave writes
            // its RW x 32*kTN block row-major (row stride skewed by 4 floats against bank
            // conflicts), then each lane owns one 32-column block of one row at a time and
            // OCP-MX quantises it alone: block maximum, 32 codes packed into 16 bytes, one
            // scale byte.
            constexpr int kLd = 32 * kTN + 4;                         // row stride (floats), skewed
            constexpr int RW = 32 * kTM;                              // rows of the wave's block
            static_assert(kNW * RW * kLd * 4 <= kStages * kStage, "epilogue staging fits the stage buffers");
            float *hq_lds = (float *)smem + wave * (RW * kLd);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = 32 * i + 8 * (v >> 2) + 4 * hb + (v & 3);
                        hq_lds[r * kLd + 32 * j + hr] = silu_fast(acc[0][i][j][v]) * acc[1][i][j][v];
                    }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // LDS is in order within a wave
            const bool vec_ok = (((uintptr_t)p.oq) & 15u) == 0;
#pragma unroll
            for (int it0 = 0; it0 < RW * kTN; it0 += 64) {
                const int rr = (it0 + lane) % RW, jb = (it0 + lane) / RW;   // row in the block, column block
                const int r = m0 + RW * wm + rr;                          // row within the expert
                const bool row_ok = r < M;
                const size_t orow = (size_t)(row0 + (row_ok ? r : 0));
                const int nb = n0 + 32 * kTN * wn + 32 * jb;              // first column of the block
                f32x4 h[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) h[q] = *(const f32x4 *)(hq_lds + rr * kLd + 32 * jb + 4 * q);
                if (!row_ok || nb >= p.N) continue;
                if (p.out) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) *(f32x4 *)(p.out + orow * p.N + nb + 4 * q) = h[q];
                }
                uint32_t amax = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q)
#pragma unroll
                    for (int c = 0; c < 4; ++c) amax = max(amax, __float_as_uint(h[q][c]) & 0x7fffffffu);
                uint32_t w[4] = {0, 0, 0, 0}, sbyte = 255;
                if (amax < 0x7f800000u) {
                    const int ebits = (int)(amax >> 23);
                    int X = ebits == 0 ? -127 : ebits - 127 - 2;
                    X = X < -127 ? -127 : (X > 127 ? 127 : X);
                    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
#pragma unroll
                    for (int q = 0; q < 8; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float x = h[q][c];
                            const uint32_t code = e2m1_code_of(fabsf(x) * inv) | ((__float_as_uint(x) >> 31) << 3);
                            w[q >> 1] |= code << (4 * (4 * (q & 1) + c));
                        }
                    sbyte = (uint32_t)(X + 127);
                }
                uint8_t *dst = p.oq + orow * (size_t)(p.N / 2) + nb / 2;
                if (vec_ok) {
                    *(u32x4 *)dst = u32x4{w[0], w[1], w[2], w[3]};
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q) dst[q] = (uint8_t)(w[q >> 2] >> (8 * (q & 3)));
                }
                p.os[orow * (size_t)(p.N / 32) + nb / 32] = (uint8_t)sbyte;
            }
        }
    }
}

// The matrix-core GEMM serves MX-quantised activations when there are enough rows per
// expert to fill 128-row tiles at least partly (prefill); decode sizes use the GEMV.
bool mfma_path_wanted(const moe_expert_weights *w, int act, int T, int k, bool routed) {
    (void)k;
    (void)routed;
    return act == MOE_ACT_MXFP4 && w->format == MOE_W_MXFP4 && T >= 64 && w->d_ff % 32 == 0 &&
           w->d_model % 32 == 0;
}

// Workgroups resident at once for a kernel on the current device (queried once per device).
template <bool PAIR, bool ROUTED>
static int resident_workgroups() {
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mxgemm_kernel<PAIR, ROUTED>, kGThreads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cache[dev] = cus * per_cu;
    }
    return cache[dev];
}

// Persistent launch: at most one wave of resident workgroups, each walking the (row tile,
// column tile) items with a stride of the grid size.  `mt_bound` bounds the row tiles.
template <bool PAIR, bool ROUTED>
static moe_status gemm_launch(const GemmParams &p, int mt_bound, hipStream_t stream, const char *what) {
    const int64_t items = (int64_t)mt_bound * ((p.N + kGBN - 1) / kGBN);
    const int64_t g = std::min<int64_t>(items, resident_workgroups<PAIR, ROUTED>());
    if (g <= 0) return MOE_OK;
    hipLaunchKernelGGL((mxgemm_kernel<PAIR, ROUTED>), dim3((unsigned)g), dim3(kGThreads), 0, stream, p);
    return launch_check(what);
}

static int tile_slots(const moe_expert_weights *w, int T, int R, bool routed) {
    if (!routed) return (T + kGBM - 1) / kGBM;
    const int ne = w->num_experts < R ? w->num_experts : R;
    return ne + R / kGBM;            // >= sum over experts of ceil(M_e / 128)
}

moe_status mfma_gateup_launch(const moe_expert_weights *w, int T, int k, const uint8_t *xq, const uint8_t *xs,
                              const int32_t *offsets, const int32_t *sorted_pairs, int R, float *h, uint8_t *hq,
                              uint8_t *hs, hipStream_t stream) {
    GemmParams p = {};
    p.a = xq;
    p.as = xs;
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
    p.oq = hq;
    p.os = hs;
    const int mt = tile_slots(w, T, R, offsets != nullptr);
    return offsets ? gemm_launch<true, true>(p, mt, stream, "moe_expert_gateup (FP4 GEMM)")
                   : gemm_launch<true, false>(p, mt, stream, "moe_expert_gateup (FP4 GEMM)");
}

moe_status mfma_down_launch(const moe_expert_weights *w, const uint8_t *hq, const uint8_t *hs, const int32_t *offsets,
                            int R, float *y, hipStream_t stream) {
    GemmParams p = {};
    p.a = hq;
    p.as = hs;
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
    const int mt = tile_slots(w, R, R, offsets != nullptr);
    return offsets ? gemm_launch<false, true>(p, mt, stream, "moe_expert_down (FP4 GEMM)")
                   : gemm_launch<false, false>(p, mt, stream, "moe_expert_down (FP4 GEMM)");
}

}  // namespace moe

// Prefill grouped GEMM on the gfx950 block-scaled FP4 matrix instructions.
//
// With MX-quantised activations both operands of every expert product are MXFP4: 32-value
// E2M1 blocks sharing one E8M0 scale (the format the pages name: rabbit README, opening
// section and architecture table).  v_mfma_scale_f32_16x16x128_f8f6f4 takes exactly that:
// lane l supplies 16 bytes (one 32-value block) of row l%16, K-block l/16, and the block's
// scale byte; it accumulates the scaled products in float32.
//
// Tile: a workgroup computes 128 rows of one expert (tokens routed to it, in sorted order)
// by 128 output columns -- of gate AND up for the SwiGLU pair.  Its 4 waves each own a
// 64 x 64 quarter as 4 x 4 MFMA tiles per matrix.  K advances in steps of 128 values.
// A step's A rows (gathered token rows), B rows (weight rows) and scale bytes travel from
// global memory straight into LDS (global_load_lds), laid out lane-major exactly as the
// MFMA reads its operands; several steps are in flight at once, so the copies of later
// steps overlap the matrix work of the current one.
// Epilogue, gate/up: h = silu(g) * u in registers, then OCP-MX quantisation of h per 32
// columns: the 16 lanes of a DPP row hold 16 consecutive columns of the same token row,
// so the block maximum is a row reduction and each lane encodes its own two values.
// Epilogue, down: float32 rows of y.
// The grid is persistent (one wave of resident workgroups); each workgroup turns
// expert_offsets into a prefix of row tiles per expert in LDS and walks its share of the
// (row tile, column tile) items, so no workgroup is launched for tiles that do not exist.
#include <algorithm>
#include <type_traits>

#include "gemv.h"

namespace moe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kGBM = 128;          // rows (tokens) per workgroup tile
constexpr int kGBN = 128;          // output columns per workgroup tile
constexpr int kGThreads = 256;

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

MOE_DEV float row16_max(float v) {
    // max over the 16 lanes of a DPP row (quad xor 1, quad xor 2, half mirror, mirror)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}
MOE_DEV uint32_t row16_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
    return v;
}

MOE_DEV uint32_t e2m1_code_of(float a) {   // same midpoint rule as the activation quantiser
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
           (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 4   // K-steps resident in LDS for gate/up (one fewer for down)
#endif
constexpr int kFrag = 1024;                    // one MFMA operand fragment: 64 lanes x 16 B

// Asynchronous global -> LDS copy (global_load_lds): lane l's bytes land at dst + 16 l
// (dst is the same in every lane; the instruction takes it from M0).  Written as asm so
// that the compiler does not add a wait for all copies in flight before every LDS read;
// the pipeline below waits for exactly the copies it needs.  The instruction has no
// register result, so nothing the compiler allocates is written when it completes.
MOE_DEV void dma16(const void *src, const unsigned char *dst) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(l) : "memory");
}
MOE_DEV void dma4(const void *src, const unsigned char *dst) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(l) : "memory");
}

// Wait until at most N of this wave's memory operations are outstanding, finish its LDS
// reads, then meet the other waves.  One asm block, so no memory access moves across it.
template <int N>
MOE_DEV void wait_vm_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}

// Row tiles per expert, as an inclusive prefix over experts in LDS: tp[e] = number of
// 128-row tiles of experts 0..e.  Every workgroup builds it once from expert_offsets.
MOE_DEV int build_tile_prefix(const int32_t *offsets, int E, int R, int *tp, int *s_wave) {
    constexpr int kPer = (MOE_MAX_EXPERTS + kGThreads - 1) / kGThreads;   // experts per thread
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    int t[kPer], sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = tid * kPer + u;
        const int lo = offsets[min(e, E)], hi = offsets[min(e + 1, E)];
        const int m = (e < E && lo >= 0 && hi <= R) ? max(hi - lo, 0) : 0;
        t[u] = (m + kGBM - 1) / kGBM;
        sum += t[u];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kGThreads / 64; ++w) {
        base += w < wave ? s_wave[w] : 0;
        total += s_wave[w];
    }
    int run = base + incl - sum;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        run += t[u];
        const int e = tid * kPer + u;
        if (e < E) tp[e] = run;
    }
    __syncthreads();
    return total;
}

// Expert owning row tile mt: the first e with tp[e] > mt (E <= 64 * 32: two probes).
MOE_DEV int tile_expert(const int *tp, int E, int mt) {
    const int lane = lane_id();
    const int probe = min(lane * 32 + 31, E - 1);
    const uint64_t m1 = __ballot(lane * 32 < E && tp[probe] > mt);
    const int c = __ffsll((long long)m1) - 1;                  // chunk of 32 experts
    const int e2 = c * 32 + (lane & 31);
    const uint64_t m2 = __ballot(lane < 32 && e2 < E && tp[min(e2, E - 1)] > mt);
    return c * 32 + __ffsll((long long)m2) - 1;
}

template <bool PAIR>
constexpr int gemm_stages() { return PAIR ? MOE_GEMM_STAGES : MOE_GEMM_STAGES - 1; }

template <bool PAIR, bool ROUTED>
__global__ __launch_bounds__(kGThreads) void mxgemm_kernel(const GemmParams p) {
    constexpr int NM = PAIR ? 2 : 1;
    constexpr int kStages = gemm_stages<PAIR>();
    constexpr int kA = 8 * kFrag;                      // A: 8 fragments of 16 rows
    constexpr int kB = NM * 8 * kFrag;                 // B: 8 fragments per matrix
    constexpr int kSRows = kGBM + NM * kGBN;           // scale rows: A, then each matrix's
    constexpr int kStage = kA + kB + kSRows * 8;       // each scale row: two aligned dwords
    constexpr int kSDma = kSRows * 2 / (64 * 4);       // scale dword copies per wave per stage
    constexpr int kOps = 2 + 2 * NM + kSDma;           // memory operations per wave per stage
    static_assert(kSRows * 2 == kSDma * 64 * 4, "scale rows must fill whole wave copies");
    static_assert(kStages >= 2 && (kStages - 2) * kOps <= 63, "vmcnt limit");
    __shared__ __align__(16) unsigned char smem[kStages * kStage];
    __shared__ uint8_t s_off[kSRows];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kGThreads / 64];

    const int NT = (p.N + kGBN - 1) / kGBN;
    const int total_mt = ROUTED ? build_tile_prefix(p.offsets, p.E, p.R, s_tp, s_wave) : (p.T + kGBM - 1) / kGBM;
    const int items = total_mt * NT;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int mt = item / NT;
        int e = 0, tile = mt, row0 = 0, M = p.T;
        if constexpr (ROUTED) {
            e = tile_expert(s_tp, p.E, mt);
            tile = mt - (e > 0 ? s_tp[e - 1] : 0);
            row0 = p.offsets[e];
            M = p.offsets[e + 1] - row0;
        }
        const int m0 = tile * kGBM;
        const int n0 = (item - mt * NT) * kGBN;
        const int lane = lane_id(), wave = wave_id();
        const int wm = wave >> 1, wn = wave & 1;       // output quarter of this wave
        const int fr = lane & 15, fg = lane >> 4;      // fragment row / K-block of this lane
        const int Kh = p.K / 2, Kb = p.K / 32;
        const int S = (Kb + 3) / 4;                    // K-steps of 128 values

        // Source row of A row r of the tile (rows past the expert's end repeat a valid row).
        auto a_src_row = [&](int r) {
            int src = row0 + min(m0 + r, M - 1);
            if (p.gather) src = p.sorted_pairs[src] / p.k;
            return min(max(src, 0), p.n_arows - 1);
        };
        auto b_src_row = [&](int n) { return (size_t)e * p.N + min(n0 + n, p.N - 1); };

        // ---- copy assignment.  Wave w copies fragments 2w and 2w+1 of A and of each B matrix:
        // lane l fetches row 16f + l%16, K-block l/16 of the step, so LDS holds every fragment
        // in the order the MFMA reads it (lane l at byte 16 l).
        const uint8_t *a_row[2], *b_row[NM][2];
    #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = 16 * (2 * wave + u) + fr;
            a_row[u] = p.a + (size_t)a_src_row(r) * Kh + fg * 16;
    #pragma unroll
            for (int mi = 0; mi < NM; ++mi) b_row[mi][u] = p.w[mi] + b_src_row(r) * Kh + fg * 16;
        }
        // Scale row q's four bytes of a step start at a fixed misalignment o within an aligned
        // dword; copying that dword and the next gives an 8-byte window holding them.  The
        // second dword is fetched only when a byte of the step lies in it (otherwise the first
        // is fetched again), so every fetched dword holds a byte of the array.
        const uint8_t *sc_row[kSDma];
        int sc_part[kSDma];
    #pragma unroll
        for (int i = 0; i < kSDma; ++i) {
            const int d = (kSDma * wave + i) * 64 + lane;
            const int q = d >> 1;
            sc_part[i] = d & 1;
            const uint8_t *row;
            if (q < kGBM) row = p.as + (size_t)a_src_row(q) * Kb;
            else if (q < kGBM + kGBN) row = p.ws[0] + b_src_row(q - kGBM) * Kb;
            else row = p.ws[NM - 1] + b_src_row(q - kGBM - kGBN) * Kb;
            sc_row[i] = row;
            if (sc_part[i] == 0) s_off[q] = (uint8_t)((uintptr_t)row & 3u);
        }
        __syncthreads();
        // Consumer side: LDS byte of each scale this lane feeds to the MFMA (step-relative).
        int sa_at[4], sb_at[NM][4];
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + 16 * i + fr;
            sa_at[i] = kA + kB + r * 8 + s_off[r] + fg;
    #pragma unroll
            for (int mi = 0; mi < NM; ++mi) {
                const int q = kGBM + mi * kGBN + wn * 64 + 16 * i + fr;
                sb_at[mi][i] = kA + kB + q * 8 + s_off[q] + fg;
            }
        }

        // Issue the copies of step s into its stage buffer (steps past the end re-fetch the
        // last step; that data is never read).
        auto issue = [&](int s) {
            const int sc = min(s, S - 1);
            unsigned char *st = smem + (s % kStages) * kStage;
            const size_t boff = (size_t)min(4 * sc + fg, Kb - 1) * 16 - (size_t)fg * 16;
    #pragma unroll
            for (int u = 0; u < 2; ++u) dma16(a_row[u] + boff, st + (2 * wave + u) * kFrag);
    #pragma unroll
            for (int mi = 0; mi < NM; ++mi)
    #pragma unroll
                for (int u = 0; u < 2; ++u) dma16(b_row[mi][u] + boff, st + kA + (mi * 8 + 2 * wave + u) * kFrag);
            const int nvalid = min(4, Kb - 4 * sc);
    #pragma unroll
            for (int i = 0; i < kSDma; ++i) {
                const uintptr_t a = (uintptr_t)(sc_row[i] + 4 * sc);
                const uintptr_t o = a & 3u;
                const uintptr_t al = a - o + ((sc_part[i] && o + nvalid > 4) ? 4u : 0u);
                dma4((const void *)al, st + kA + kB + (kSDma * wave + i) * 256);
            }
        };

        f32x4 acc[NM][4][4];
    #pragma unroll
        for (int mi = 0; mi < NM; ++mi)
    #pragma unroll
            for (int i = 0; i < 4; ++i)
    #pragma unroll
                for (int j = 0; j < 4; ++j) acc[mi][i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        // One K-step of matrix work from stage buffer st.  TAIL: the last step when K is not a
        // multiple of 128 -- K-blocks past the end get zero A codes and unit scales.
        auto compute = [&](const unsigned char *st, auto tail) {
            constexpr bool TAIL = decltype(tail)::value;
            const bool dead = TAIL && 4 * (S - 1) + fg >= Kb;
            i32x8_t af[4];
            int asc[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = *(const u32x4 *)(st + (wm * 4 + i) * kFrag + lane * 16);
                af[i] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
                asc[i] = (int)st[sa_at[i]];
                if constexpr (TAIL) {
                    af[i] = dead ? i32x8_t{0, 0, 0, 0, 0, 0, 0, 0} : af[i];
                    asc[i] = dead ? 127 : asc[i];
                }
            }
    #pragma unroll
            for (int mi = 0; mi < NM; ++mi) {
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 v = *(const u32x4 *)(st + kA + (mi * 8 + wn * 4 + j) * kFrag + lane * 16);
                    const i32x8_t bf = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
                    int bsc = (int)st[sb_at[mi][j]];
                    if constexpr (TAIL) bsc = dead ? 127 : bsc;
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mi][i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[mi][i][j], 4, 4, 0,
                                                                                       asc[i], 0, bsc);
                }
            }
        };

    #pragma unroll
        for (int s = 0; s < kStages - 1; ++s) issue(s);
        const int S_full = (Kb & 3) ? S - 1 : S;           // steps with four whole K-blocks
        for (int s = 0; s < S; ++s) {
            // this wave's copies of step s are done once at most the later stages' are pending
            wait_vm_and_barrier<(kStages - 2) * kOps>();
            issue(s + kStages - 1);                        // into the buffer read at step s-1
            const unsigned char *st = smem + (s % kStages) * kStage;
            if (s < S_full) compute(st, std::false_type{});
            else compute(st, std::true_type{});
        }
        wait_vm_and_barrier<0>();                          // no copy in flight at exit

        // ---- epilogue.  Lane holds C[4*fg + v][fr] of each 16x16 tile.
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
    #pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = m0 + wm * 64 + 16 * i + 4 * fg + v;      // row within the expert
                const bool row_ok = r < M;
                const size_t orow = (size_t)(row0 + (row_ok ? r : 0));
                float val[4];
    #pragma unroll
                for (int j = 0; j < 4; ++j) val[j] = PAIR ? silu(acc[0][i][j][v]) * acc[NM - 1][i][j][v] : acc[0][i][j][v];
                // float32 output (y, or h when requested)
                if (p.out) {
    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = n0 + wn * 64 + 16 * j + fr;
                        if (row_ok && n < p.N) p.out[orow * p.N + n] = val[j];
                    }
                }
                if constexpr (PAIR) {
                    // MX quantisation per 32 columns: tiles (j, j+1) = columns [32q, 32q+32) of the quarter
    #pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const float x0 = val[2 * q], x1 = val[2 * q + 1];
                        const uint32_t a0 = __float_as_uint(x0) & 0x7fffffffu, a1 = __float_as_uint(x1) & 0x7fffffffu;
                        const uint32_t amax = row16_max_u32(max(a0, a1));
                        uint32_t c0 = 0, c1 = 0, sbyte = 255;
                        if (amax < 0x7f800000u) {
                            const int ebits = (int)(amax >> 23);
                            int X = ebits == 0 ? -127 : ebits - 127 - 2;
                            X = X < -127 ? -127 : (X > 127 ? 127 : X);
                            const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
                            c0 = e2m1_code_of(fabsf(x0) * inv) | ((__float_as_uint(x0) >> 31) << 3);
                            c1 = e2m1_code_of(fabsf(x1) * inv) | ((__float_as_uint(x1) >> 31) << 3);
                            sbyte = (uint32_t)(X + 127);
                        }
                        // element n of the 32-block: tile 2q holds n = fr, tile 2q+1 holds n = 16 + fr;
                        // byte b = (n/2) packs elements 2b (low nibble) and 2b+1 (high nibble)
                        const uint32_t o0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)c0, 0xB1, 0xF, 0xF, false);
                        const uint32_t o1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)c1, 0xB1, 0xF, 0xF, false);
                        const int nb = n0 + wn * 64 + 32 * q;              // first column of the block
                        if (row_ok && nb < p.N && (fr & 1) == 0) {
                            uint8_t *dst = p.oq + orow * (size_t)(p.N / 2) + nb / 2;
                            dst[fr / 2] = (uint8_t)(c0 | (o0 << 4));
                            dst[8 + fr / 2] = (uint8_t)(c1 | (o1 << 4));
                        }
                        if (row_ok && nb < p.N && fr == 0) p.os[orow * (size_t)(p.N / 32) + nb / 32] = (uint8_t)sbyte;
                    }
                }
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

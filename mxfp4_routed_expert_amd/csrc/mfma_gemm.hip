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
// 64 x 64 quarter as 4 x 4 MFMA tiles per matrix.  K advances in steps of 128 values:
// the workgroup stages the step's A rows (gathered token rows), B rows (weight rows) and
// their scale bytes in LDS (rows padded to 80 bytes against bank conflicts), while the
// next step's data is already loading into registers.
// Epilogue, gate/up: h = silu(g) * u in registers, then OCP-MX quantisation of h per 32
// columns: the 16 lanes of a DPP row hold 16 consecutive columns of the same token row,
// so the block maximum is a row reduction and each lane encodes its own two values.
// Epilogue, down: float32 rows of y.
// Which (expert, 128-row tile) a workgroup owns comes from expert_offsets on the device.
#include "gemv.h"

namespace moe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kGBM = 128;          // rows (tokens) per workgroup tile
constexpr int kGBN = 128;          // output columns per workgroup tile
constexpr int kGThreads = 256;
constexpr int kGRowPad = 80;       // LDS bytes per staged row (64 data + 16 pad)

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

// The b-th (expert, row tile) of the routed rows: returns the expert (or -1) and the tile.
MOE_DEV int wave_nth_tile(const int32_t *offsets, int E, int b, int *tile) {
    const int lane = lane_id();
    int o[kMaxOffsetChunks];
#pragma unroll
    for (int c = 0; c < kMaxOffsetChunks; ++c) o[c] = offsets[min(c * 64 + lane, E)];
    int base = 0;
#pragma unroll
    for (int c = 0; c < kMaxOffsetChunks; ++c) {
        if (c * 64 >= E) break;
        const int next = c + 1 < kMaxOffsetChunks ? __shfl(o[c + 1], 0, kWave) : 0;
        int o1 = __shfl_down(o[c], 1, kWave);
        if (lane == 63) o1 = next;
        const int e = c * 64 + lane;
        const int m = e < E ? max(o1 - o[c], 0) : 0;
        const int tiles = (m + kGBM - 1) / kGBM;
        int incl = tiles;            // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, 63, kWave);
        if (b < base + total) {
            const bool mine = tiles > 0 && b >= base + incl - tiles && b < base + incl;
            const uint64_t hit = __ballot(mine);
            const int L = __ffsll((long long)hit) - 1;
            *tile = b - (base + __shfl(incl, L, kWave) - __shfl(tiles, L, kWave));
            return c * 64 + L;
        }
        base += total;
    }
    return -1;
}

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

template <bool PAIR, bool ROUTED>
__global__ __launch_bounds__(kGThreads) void mxgemm_kernel(const GemmParams p) {
    constexpr int NM = PAIR ? 2 : 1;
    __shared__ __align__(16) unsigned char sA[kGBM * kGRowPad];
    __shared__ __align__(16) unsigned char sB[NM][kGBN * kGRowPad];
    __shared__ uint32_t sSA[kGBM];
    __shared__ uint32_t sSB[NM][kGBN];

    int e = 0, tile = blockIdx.y, row0 = 0, M = p.T;
    if constexpr (ROUTED) {
        e = wave_nth_tile(p.offsets, p.E, blockIdx.y, &tile);
        if (e < 0) return;
        row0 = p.offsets[e];
        M = p.offsets[e + 1] - row0;
        if (row0 < 0 || M <= 0 || row0 + M > p.R) return;
    }
    const int m0 = tile * kGBM;
    if (m0 >= M) return;
    const int n0 = blockIdx.x * kGBN;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;       // wave quarter
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (Kb + 3) / 4;                    // K-steps of 128 values

    // ---- per-thread staging assignment: A row chunk(s), B row chunks, scale rows
    // A: 128 rows x 4 chunks of 16 B = 512 chunks -> 2 per thread; B: same per matrix.
    const uint8_t *arow[2];
    int achunk[2], arow_i[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + kGThreads * i;
        const int r = c >> 2;
        achunk[i] = c & 3;
        arow_i[i] = r;
        const int rr = min(m0 + r, M - 1);             // rows past the expert's end repeat a valid row
        int src = row0 + rr;
        if (p.gather) src = p.sorted_pairs[src] / p.k;
        src = min(max(src, 0), p.n_arows - 1);
        arow[i] = p.a + (size_t)src * Kh;
    }
    const uint8_t *brow[NM][2];
    int bchunk[2], brow_i[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + kGThreads * i;
        brow_i[i] = c >> 2;
        bchunk[i] = c & 3;
        const int n = min(n0 + (c >> 2), p.N - 1);
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) brow[mi][i] = p.w[mi] + ((size_t)e * p.N + n) * Kh;
    }
    // scale rows: threads 0..127 -> A row tid; threads 128..255 -> B row tid-128 (each matrix).
    // Every thread gets valid pointers for both roles and picks with a select, so the scale
    // loads below are unconditional (a load under a branch is waited for at the join).
    const uint8_t *sp0, *sp1;
    {
        const int rr = min(m0 + (tid & (kGBM - 1)), M - 1);
        int src = row0 + rr;
        if (p.gather) src = p.sorted_pairs[src] / p.k;
        src = min(max(src, 0), p.n_arows - 1);
        const uint8_t *sa = p.as + (size_t)src * Kb;
        const int n = min(n0 + (tid & (kGBN - 1)), p.N - 1);
        const uint8_t *sb0 = p.ws[0] + ((size_t)e * p.N + n) * Kb;
        const uint8_t *sb1 = p.ws[NM - 1] + ((size_t)e * p.N + n) * Kb;
        sp0 = tid < kGBM ? sa : sb0;
        sp1 = tid < kGBM ? sa : sb1;
    }

    u32x4 ra[2], rb[NM][2];
    uint32_t rs0 = 0, rs1 = 0;
    auto gload = [&](int s) {
        // unconditional loads from clamped positions; blocks past K are zeroed at the store
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int blk = min(4 * s + achunk[i], Kb - 1);
            ra[i] = __builtin_nontemporal_load((const u32x4 *)(arow[i] + (size_t)blk * 16));
        }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int blk = min(4 * s + bchunk[i], Kb - 1);
                rb[mi][i] = __builtin_nontemporal_load((const u32x4 *)(brow[mi][i] + (size_t)blk * 16));
            }
        uint32_t v0[4], v1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int blk = min(4 * s + q, Kb - 1);
            v0[q] = sp0[blk];
            if constexpr (PAIR) v1[q] = sp1[blk];
        }
        uint32_t s0 = 0, s1 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = 4 * s + q < Kb;
            s0 |= (ok ? v0[q] : 127u) << (8 * q);
            if constexpr (PAIR) s1 |= (ok ? v1[q] : 127u) << (8 * q);
        }
        rs0 = s0;
        rs1 = s1;
    };
    auto lstore = [&](int s) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bool ok = 4 * s + achunk[i] < Kb;
            *(u32x4 *)(sA + arow_i[i] * kGRowPad + achunk[i] * 16) = ok ? ra[i] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bool ok = 4 * s + bchunk[i] < Kb;
                *(u32x4 *)(sB[mi] + brow_i[i] * kGRowPad + bchunk[i] * 16) = ok ? rb[mi][i] : u32x4{0, 0, 0, 0};
            }
        if (tid < kGBM) {
            sSA[tid] = rs0;
        } else {
            sSB[0][tid - kGBM] = rs0;
            if constexpr (PAIR) sSB[NM - 1][tid - kGBM] = rs1;
        }
    };

    f32x4 acc[NM][4][4];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mi][i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = lane & 15, fg = lane >> 4;      // fragment row / K-block of this lane
    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) gload(s + 1);
        i32x8_t af[4];
        int asc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + 16 * i + fr;
            const u32x4 v = *(const u32x4 *)(sA + r * kGRowPad + fg * 16);
            af[i] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
            asc[i] = (int)((sSA[r] >> (8 * fg)) & 0xffu);
        }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wn * 64 + 16 * j + fr;
                const u32x4 v = *(const u32x4 *)(sB[mi] + n * kGRowPad + fg * 16);
                const i32x8_t bf = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
                const int bsc = (int)((sSB[mi][n] >> (8 * fg)) & 0xffu);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[mi][i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf, acc[mi][i][j], 4, 4, 0,
                                                                                   asc[i], 0, bsc);
            }
        }
        __syncthreads();
        if (s + 1 < S) {
            lstore(s + 1);
            __syncthreads();
        }
    }

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

// The matrix-core GEMM serves MX-quantised activations when there are enough rows per
// expert to fill 128-row tiles at least partly (prefill); decode sizes use the GEMV.
bool mfma_path_wanted(const moe_expert_weights *w, int act, int T, int k, bool routed) {
    (void)k;
    (void)routed;
    return act == MOE_ACT_MXFP4 && w->format == MOE_W_MXFP4 && T >= 64 && w->d_ff % 32 == 0 &&
           w->d_model % 32 == 0;
}

static moe_status gemm_launch(GemmParams p, bool pair, int slots, hipStream_t stream, const char *what) {
    dim3 grid((p.N + kGBN - 1) / kGBN, slots);
    auto fn = pair ? (p.offsets ? mxgemm_kernel<true, true> : mxgemm_kernel<true, false>)
                   : (p.offsets ? mxgemm_kernel<false, true> : mxgemm_kernel<false, false>);
    hipLaunchKernelGGL(fn, grid, dim3(kGThreads), 0, stream, p);
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
    return gemm_launch(p, true, tile_slots(w, T, R, offsets != nullptr), stream, "moe_expert_gateup (FP4 GEMM)");
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
    return gemm_launch(p, false, tile_slots(w, R, R, offsets != nullptr), stream, "moe_expert_down (FP4 GEMM)");
}

}  // namespace moe

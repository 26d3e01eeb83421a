// Prefill grouped GEMM on the gfx950 block-scaled FP4 matrix instructions.
//
// With MX-quantised activations both operands of every expert product are MXFP4: 32-value
// E2M1 blocks sharing one E8M0 scale (the format the pages name: rabbit README, opening
// section and architecture table).  v_mfma_scale_f32_32x32x64_f8f6f4 takes exactly that:
// lane l supplies 16 bytes (one 32-value block) of row l%32 and K-group l/32, plus a 32-bit
// register whose byte `opsel` is the block's scale; it accumulates the scaled products in
// float32.  The K order inside a product is free as long as both operands use the same one,
// so lane group g takes blocks 4g .. 4g+3 of each 256-value K-step, one per quarter q: the
// four scale bytes a lane needs in a step are one dword, and quarter q selects byte q.
//
// Item: 256 rows of one expert (tokens routed to it, in sorted order) by 256 weight rows
// (128 columns of gate AND of up for the SwiGLU pair; 256 output columns for down).  One
// workgroup of 8 waves per CU, two waves per SIMD; wave (wm, wn) owns 128 rows x 2 weight
// tiles of 32 (a gate and an up tile of the same 32 columns for the pair, 64 output
// columns for down), i.e. 8 accumulator tiles (128 registers).
// K advances in steps of 256 values: every operand row contributes one whole 128-byte
// line per step.  A step's A rows (gathered token rows), B rows (weight rows) and scale
// windows go from global memory straight into LDS (global_load_lds), two steps resident
// (2 x 72 KB); every wave issues an eighth of the next step's copies between its matrix
// instructions of the current step.  A wave stalls while the L1 accepts its copies (the
// copy rate grows with the number of waves issuing), so the second wave on each SIMD keeps
// the matrix core busy meanwhile.
// Small row counts: an item whose live rows fit 128 (or 64) runs with 2 (or 1) row tiles
// per wave, so all eight waves share the smaller tile; and when the last round of items
// would leave CUs idle, its items are split into halves or quarters by rows.
// Epilogue, gate/up: h = silu(g) * u, staged through LDS so that each lane owns a row's
// 32-column block and OCP-MX quantises it alone (block maximum, 16 packed code bytes, one
// scale byte).  Epilogue, down: float32 rows of y.
// The grid is persistent (one workgroup per CU); each workgroup turns expert_offsets into a
// prefix of 256-row tiles per expert in LDS and walks its share of the work units.
#include <algorithm>
#include <type_traits>

#include "gemv.h"
#include "tile_sched.h"

namespace moe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kQBM = 256;              // rows per item
constexpr int kQBR = 256;              // weight rows per item
constexpr int kQThreads = 512;         // 8 waves, 2 along the rows x 4 along the weight rows
constexpr int kQRowB = 128;            // code bytes per row per K-step (256 values)
constexpr int kQSlot = 16;             // LDS bytes per scale row per step
// LDS: A codes of both stages, then B codes of both stages, then scale windows of both.
constexpr int kQA = kQBM * kQRowB;                   // 32 KB per stage
constexpr int kQB = kQBR * kQRowB;                   // 32 KB per stage
constexpr int kQS = (kQBM + kQBR) * kQSlot;          // 8 KB per stage
constexpr int kQOffA = 0, kQOffB = 2 * kQA, kQOffS = 2 * kQA + 2 * kQB;
constexpr int kQLds = kQOffS + 2 * kQS;              // 144 KB
constexpr int kQLd = 32 + 4;                         // epilogue staging row stride (floats)
static_assert(8 * 128 * kQLd * 4 <= kQLds, "epilogue staging fits the stage buffers");

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

// Asynchronous global -> LDS copy (global_load_lds): lane l reads base + voff and its bytes
// land at dst + l * size (dst is the same in every lane; the instruction takes it from M0).
// Written as asm so that the compiler does not add a wait for all copies in flight before
// every LDS read; the pipeline below waits for exactly the copies it needs.  The
// instruction has no register result, so nothing the compiler allocates is written when
// it completes.
MOE_DEV void dma16(const uint8_t *base, uint32_t voff, const unsigned char *dst) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(l) : "memory");
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

// All of this wave's copies have landed and its LDS reads are done; then the waves meet.
// One asm block, so no memory access moves across it.
MOE_DEV void wait_copies_and_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The lane id, read so that the compiler neither hoists it nor keeps values derived from it
// alive across a loop.
MOE_DEV int lane_fresh() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Position of 16-byte chunk c of LDS row r is c ^ qswz(r): a quarter's operand read (rows
// r .. r+31 at one chunk) then spreads over all 16-byte bank groups whether the banks repeat
// every 128 or every 256 bytes.
MOE_DEV int qswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// One unit of work: rows [m0, m0 + live) of expert e (row0 = its first sorted row, M its
// row count) against weight rows n0 .. n0+127 of gate and up (pair) or n0 .. n0+255 (down).
struct QUnit {
    int e, n0, m0, row0, M;
};

template <bool PAIR, int TM, bool AS>
MOE_DEV void qgemm_unit(const GemmParams &p, const QUnit &u, unsigned char *smem, const int *s_arow) {
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave >> 2, wn = wave & 3;
    const int hr = lane & 31, hb = lane >> 5;
    const int Kh = p.K / 2, Kb = p.K / 32;
    const int S = (Kb + 7) / 8;                   // K-steps
    const int nvalid = Kb - 8 * (S - 1);          // blocks of the last step (1..8)
    const int eu = __builtin_amdgcn_readfirstlane(u.e);

    // ---- copy sources.  A: the unit's 64*TM rows, 8*TM per wave: rows wave*8*TM + 8t + lane/8
    // (t < TM; LDS rows in that order), lane%8 = the LDS chunk position, fetching chunk
    // (lane%8) ^ qswz(row).
    const uint8_t *a_base = uniform_ptr(p.a);
    const uint8_t *as_base = uniform_ptr((const uint8_t *)((uintptr_t)p.as & ~(uintptr_t)3));
    const uint32_t as_mis = (uint32_t)((uintptr_t)p.as & 3u);
    // B: wave w copies LDS B rows 32w .. 32w+31: for the pair, gate rows n0 + 32w + .. (w < 4)
    // or up rows n0 + 32(w-4) + .. (w >= 4); for down, rows n0 + 32w + ...
    const int bmat = PAIR ? (wave >> 2) : 0;
    const int bl0 = PAIR ? 32 * (wave & 3) : 32 * wave;        // first matrix row (past n0) it copies
    const uint8_t *b_base = uniform_ptr((PAIR && bmat ? p.w[1] : p.w[0]) + (size_t)eu * p.N * Kh);
    const int cr = lane >> 3, cpos = lane & 7;
    uint32_t aoff[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int r = wave * 8 * TM + 8 * t + cr;
        aoff[t] = (uint32_t)s_arow[r] * Kh + 16 * (cpos ^ qswz(r));
    }
    // B source of piece t, computed when it is issued: matrix row min(brow0 + 8t, N-1), chunk
    // (lane%8) ^ qswz(LDS row)
    const int brow0 = u.n0 + bl0 + cr;
    auto boff = [&](int t) {
        return (uint32_t)min(brow0 + 8 * t, p.N - 1) * Kh + 16 * (cpos ^ qswz(32 * wave + 8 * t + cr));
    };
    // Scale windows.  LDS scale row q (A rows 0..255, then B rows 0..255) has a 16-byte slot
    // per stage; wave w copies scale rows 64w .. 64w+63.
    //  * AS (every scale row starts on a dword: K % 128 == 0, aligned bases, K >= 512): one
    //    lane per row copies a two-step window, the row's bytes min(16j, Kb-16) .. +15 for
    //    steps 2j and 2j+1, into the slots of stage j % 2 -- one copy per wave every other step.
    //  * otherwise: every step, the aligned dwords covering the step's 8 bytes of the row, from
    //    byte 0 of the slot; 4 lanes per row, dword d of the window.  A dword past the step's
    //    bytes fetches the window's first dword again, so every fetched dword lies inside the
    //    array.
    const uint8_t *sc_base;
    uint32_t sc_rel[AS ? 1 : 4];                  // scale row start (- aligned base), per copy
    {
        const bool arows = wave < 4;
        const uint8_t *bs = PAIR && wave >= 6 ? p.ws[1] : p.ws[0];
        const uintptr_t bsa = (uintptr_t)bs & ~(uintptr_t)3;
        sc_base = uniform_ptr(arows ? (const uint8_t *)as_base : (const uint8_t *)(bsa + (size_t)eu * p.N * Kb));
        const uint32_t bmis = (uint32_t)((uintptr_t)bs & 3u);
#pragma unroll
        for (int i = 0; i < (AS ? 1 : 4); ++i) {
            const int q = AS ? 64 * wave + lane : 64 * wave + 16 * i + (lane >> 2);
            if (arows) {
                sc_rel[i] = as_mis + (uint32_t)s_arow[q] * Kb;
            } else {
                const int br = q - 256;                            // B row of the item
                const int n = PAIR ? u.n0 + (br & 127) : u.n0 + br;
                sc_rel[i] = bmis + (uint32_t)min(n, p.N - 1) * Kb;
            }
        }
    }
    const int sd = lane & 3;
    // window dword offset of this lane for a window of `len` bytes
    auto sc_voff = [&](uint32_t rel, int len) {
        const uint32_t o = rel & 3u;
        const uint32_t need = (o + (uint32_t)len - 1u) >> 2;
        return rel - o + ((uint32_t)sd <= need ? 4u * sd : 0u);
    };
    auto win_start = [&](int j) { return min(16 * j, Kb - 16); };   // AS: first byte of window j

    // Copies of step s into stage s % 2 (a step past the last copies the last step's bytes into
    // the stage no step reads any more), as 12 pieces per wave: 0-3 A codes (pieces past the
    // TM this unit needs repeat its first one: same bytes to the same place, so every step
    // issues the same number), 4-7 B codes, 8-11 scale windows.  In the last step, chunks
    // past the end of a row are clamped to its last block (read, never used) and the scale
    // windows shrink.
    auto issue_piece = [&](int s_in, int pc) {
        const int s = min(s_in, S - 1);           // past the last step: its bytes again (never read)
        const bool last = s == S - 1;
        const int st = s_in & 1;
        const uint32_t cmax = 16u * (uint32_t)(Kb - 1 - 8 * s);   // last valid chunk (bytes) in the step
        if (pc < 4) {
            const int t = pc < TM ? pc : 0;
            uint32_t v = aoff[t];
            if (last) {                           // the chunk's byte offset within the row's step line
                const uint32_t c = 16u * (uint32_t)(cpos ^ qswz(wave * 8 * TM + 8 * t + cr));
                v = v - c + min(c, cmax);
            }
            dma16(a_base + 128 * s, v, smem + kQOffA + st * kQA + wave * 8 * TM * kQRowB + t * 1024);
        } else if (pc < 8) {
            const int t = pc - 4;
            uint32_t v = boff(t);
            if (last) {
                const uint32_t c = 16u * (uint32_t)(cpos ^ qswz(32 * wave + 8 * t + cr));
                v = v - c + min(c, cmax);
            }
            dma16(b_base + 128 * s, v, smem + kQOffB + st * kQB + 32 * wave * kQRowB + t * 1024);
        } else if constexpr (AS) {
            if ((s_in & 1) || s_in >= S) return;  // a window serves steps s_in and s_in + 1
            const int j = s_in >> 1;
            dma16(sc_base + win_start(j), sc_rel[0], smem + kQOffS + (j & 1) * kQS + 64 * wave * kQSlot);
        } else {
            const int i = pc - 8;
            dma4(sc_base + 8 * s, sc_voff(sc_rel[i], last ? nvalid : 8),
                 smem + kQOffS + st * kQS + 64 * wave * kQSlot + i * 256);
        }
    };
    constexpr int kPieces = AS ? 9 : 12;

    // ---- consumer side.  Row tiles of this wave: rows 32*TM*wm + 32i (i < TM) of the unit;
    // weight tiles jb < 2: the pair's gate columns 32wn (jb = 0) and up columns 32wn (jb = 1);
    // down: columns 64wn + 32jb.  Operand address of tile x in quarter q: row base + chunk
    // (4hb + q) ^ swz = (4hb ^ swz) ^ q.
    // Tile i's rows are 32i past tile 0's, with the same low bits (so the same swizzle): its
    // operand and scale addresses are tile 0's plus a constant.  The scale bytes' offset within
    // their dword (the window starts at an aligned dword) is kept per tile in 4 bits: A tile i at
    // bit 4i, B tile jb at bit 16 + 4jb.
    // The four base addresses are recomputed at every step from a lane id the compiler cannot
    // hoist (the step loop has no registers to spare for them).
    const int ra = 32 * TM * wm + hr;
    constexpr int kBTile = PAIR ? 128 : 32;        // LDS B rows between the wave's two weight tiles
    const int rb = PAIR ? 32 * wn + hr : 64 * wn + hr;
    struct Bases {
        int a, b, sa, sb;
    };
    auto bases = [&]() {
        const int ln = lane_fresh(), hr_ = ln & 31, hb_ = ln >> 5;
        const int ra_ = 32 * TM * wm + hr_, rb_ = (PAIR ? 32 : 64) * wn + hr_;
        return Bases{kQOffA + ra_ * kQRowB + (((4 * hb_) ^ qswz(ra_)) << 4),
                     kQOffB + rb_ * kQRowB + (((4 * hb_) ^ qswz(rb_)) << 4), kQOffS + ra_ * kQSlot + 4 * hb_,
                     kQOffS + (kQBM + rb_) * kQSlot + 4 * hb_};
    };
    uint32_t so_pack = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) so_pack |= ((as_mis + (uint32_t)s_arow[ra + 32 * i] * Kb) & 3u) << (4 * i);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const uint8_t *bs = PAIR && jb == 1 ? p.ws[1] : p.ws[0];
        const int n = PAIR ? u.n0 + 32 * wn + hr : u.n0 + 64 * wn + 32 * jb + hr;
        so_pack |= ((uint32_t)(((uintptr_t)bs & 3u) + ((size_t)eu * p.N + min(n, p.N - 1)) * Kb) & 3u) << (16 + 4 * jb);
    }

    f32x16 acc[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][jb][v] = 0.0f;

    auto lds16 = [&](int addr) { return *(const u32x4 *)(smem + addr); };
    auto scale4 = [&](int addr, uint32_t o) {     // 4 scale bytes from byte o of a two-dword window
        const uint32_t d0 = *(const uint32_t *)(smem + addr), d1 = *(const uint32_t *)(smem + addr + 4);
        return __builtin_amdgcn_alignbyte(d1, d0, o);
    };

    // One K-step from stage s % 2.  In the last step, blocks past K (4hb + q >= nvalid) get
    // scale byte 0 on both operands: each of their products is at most 36 * 2^-254 in
    // magnitude, far below float32's smallest subnormal (2^-149), so it adds an exact zero
    // (their codes are real codes of a clamped block, never NaN or infinite: E2M1 has none).
    // The copies of step s+1 go out during the first half of step s's products, a piece after
    // every product or so.
    auto step = [&](int s) {
        const int so = s & 1;
        const Bases bs = bases();
        const int a_at = bs.a, b_at = bs.b, sa_at = bs.sa, sb_at = bs.sb;

        uint32_t sa[TM], sb[2];
        if constexpr (AS) {
            // the step's bytes sit at 8s - win_start(s/2) in the window; a dword wholly past K
            // (offset 16) is never needed (its blocks get scale 0 below), so it reads byte 12
            const int j = s >> 1;
            const int o = min(8 * s - win_start(j) + 4 * hb, 12) - 4 * hb;
            const int sw = (j & 1) * kQS + o;
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = *(const uint32_t *)(smem + sa_at + 32 * i * kQSlot + sw);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) sb[jb] = *(const uint32_t *)(smem + sb_at + kBTile * jb * kQSlot + sw);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = scale4(sa_at + 32 * i * kQSlot + so * kQS, (so_pack >> (4 * i)) & 3u);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                sb[jb] = scale4(sb_at + kBTile * jb * kQSlot + so * kQS, (so_pack >> (16 + 4 * jb)) & 3u);
        }
        if (s == S - 1) {
            uint32_t kmask = 0xffffffffu;          // bytes of this lane's valid quarters
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (4 * hb + q >= nvalid) kmask &= ~(0xffu << (8 * q));
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] &= kmask;
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) sb[jb] &= kmask;
        }
        u32x4 fa[2][TM], fb[2][2];
        auto rd = [&](int q, u32x4 (&a)[TM], u32x4 (&b)[2]) {
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = lds16((a_at ^ (q << 4)) + 32 * i * kQRowB + so * kQA);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) b[jb] = lds16((b_at ^ (q << 4)) + kBTile * jb * kQRowB + so * kQB);
        };
        // quarter Q: the next quarter's operands are read while this one's products run
        auto quarter = [&](auto q_c) {
            constexpr int Q = decltype(q_c)::value;
            if constexpr (Q < 3) rd(Q + 1, fa[(Q + 1) & 1], fb[(Q + 1) & 1]);
            constexpr int NH = 4 * TM;             // products in the first half of the step
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const u32x4 av = fa[Q & 1][i], bv = fb[Q & 1][jb];
                    acc[i][jb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        i32x8_t{(int)av[0], (int)av[1], (int)av[2], (int)av[3], 0, 0, 0, 0},
                        i32x8_t{(int)bv[0], (int)bv[1], (int)bv[2], (int)bv[3], 0, 0, 0, 0}, acc[i][jb], 4, 4, Q,
                        (int)sa[i], Q, (int)sb[jb]);
                    if constexpr (Q < 2) {
                        const int m = Q * 2 * TM + 2 * i + jb;
#pragma unroll
                        for (int pc = m * kPieces / NH; pc < (m + 1) * kPieces / NH; ++pc) issue_piece(s + 1, pc);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
        };
        rd(0, fa[0], fb[0]);
        quarter(std::integral_constant<int, 0>{});
        quarter(std::integral_constant<int, 1>{});
        quarter(std::integral_constant<int, 2>{});
        quarter(std::integral_constant<int, 3>{});
    };

    // ---- pipeline: two stages.  At the top of step s its copies have landed and every wave
    // is done with step s-1, whose stage takes the copies of step s+1 during step s.
#pragma unroll
    for (int pc = 0; pc < kPieces; ++pc) issue_piece(0, pc);
    for (int s = 0; s < S; ++s) {
        wait_copies_and_barrier();
        step(s);                                  // issues the copies of step s + 1 as it goes
    }
    wait_copies_and_barrier();                    // no copy in flight past this point
    __syncthreads();                              // every wave is done with the stages

    // ---- epilogue.  Lane l holds C[8(v/4) + 4(l/32) + v%4][l%32] of each 32x32 tile.
    const int rbase = u.m0 + 32 * TM * wm;        // first row (within the expert) of this wave
    if constexpr (!PAIR) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = rbase + 32 * i + 8 * (v >> 2) + 4 * hb + (v & 3);
                if (r >= u.M) continue;
                const size_t orow = (size_t)(u.row0 + r);
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const int n = u.n0 + 64 * wn + 32 * jb + hr;
                    if (n < p.N) p.out[orow * p.N + n] = acc[i][jb][v];
                }
            }
    } else {
        // h = silu(g) * u of the wave's 32*TM rows x 32 columns into LDS (row stride kQLd,
        // skewed against bank conflicts), then each lane quantises one row's 32-column block:
        // block maximum, 32 codes packed into 16 bytes, one scale byte.
        float *hq_lds = (float *)smem + wave * (128 * kQLd);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + 4 * hb + (v & 3);
                hq_lds[r * kQLd + hr] = silu_fast(acc[i][0][v]) * acc[i][1][v];
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // LDS is in order within a wave
        const bool vec_ok = (((uintptr_t)p.oq) & 15u) == 0;
        const int nb = u.n0 + 32 * wn;                         // first column of the wave's block
#pragma unroll
        for (int it0 = 0; it0 < 32 * TM; it0 += 64) {
            const int rr = it0 + lane;                         // row in the wave's block
            if (rr >= 32 * TM) continue;
            f32x4 h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = *(const f32x4 *)(hq_lds + rr * kQLd + 4 * q);
            const int r = rbase + rr;
            if (r >= u.M || nb >= p.N) continue;
            const size_t orow = (size_t)(u.row0 + r);
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

// One workgroup per CU (its LDS takes 147 KB) of 8 waves, two per SIMD: each wave may use
// half a SIMD's register file, 256 registers, of which the 8 accumulator tiles take 128.
template <bool PAIR, bool ROUTED, bool AS>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mxgemm_kernel(
    const GemmParams p) {
    __shared__ __align__(16) unsigned char smem[kQLds];
    __shared__ int s_tp[ROUTED ? MOE_MAX_EXPERTS : 1];
    __shared__ int s_wave[kQThreads / 64];
    __shared__ int s_arow[kQBM];

    const int NB = PAIR ? kQBR / 2 : kQBR;                  // output columns per item
    const int NT = (p.N + NB - 1) / NB;
    const int total_mt = ROUTED ? build_tile_prefix<kQThreads, kQBM>(p.offsets, p.E, p.R, s_tp, s_wave)
                                : (p.T + kQBM - 1) / kQBM;
    const int items = total_mt * NT;
    // Work units: whole items while they fill rounds of G workgroups; the items of a last,
    // partial round are split by rows into f parts (f = 2 or 4, as many as the idle
    // workgroups allow), so that round takes a fraction of an item's time.
    const int G = gridDim.x;
    const int full = items / G * G, tail = items - full;
    const int f = tail > 0 && 4 * tail <= G ? 4 : (tail > 0 && 2 * tail <= G ? 2 : 1);
    const int units = full + f * tail;
    // Each round of G workgroups hands XCD x (workgroups x, x+8, ...) a contiguous run of G/8
    // units: units are ordered expert by expert, then by column tile, then by row tile (and
    // part), so the row tiles that share a column tile of weights run at the same time on the
    // same XCD and take those weight bytes from its L2.
    const int slot = xcd_slot(blockIdx.x, G);

    for (int un = slot; un < units; un += G) {
        int item = un, part = 0, nparts = 1;
        if (un >= full) {
            item = full + (un - full) / f;
            part = (un - full) % f;
            nparts = f;
        }
        QUnit u;
        int tile = 0, nt = 0;
        u.e = 0;
        u.row0 = 0;
        u.M = p.T;
        if constexpr (ROUTED) {
            u.e = tile_expert(s_tp, p.E, item / NT);
            const int tpx = u.e > 0 ? s_tp[u.e - 1] : 0, te = s_tp[u.e] - tpx;
            const int r = item - NT * tpx;
            nt = r / te;
            tile = r - nt * te;
            u.row0 = p.offsets[u.e];
            u.M = p.offsets[u.e + 1] - u.row0;
        } else {
            nt = item / total_mt;
            tile = item - nt * total_mt;
        }
        const int plen = kQBM / nparts;
        u.m0 = tile * kQBM + part * plen;
        u.n0 = nt * NB;
        const int live = min(u.M - u.m0, plen);
        if (live <= 0) continue;                             // a part past the expert's last row
        const int TM = __builtin_amdgcn_readfirstlane(live > 128 ? 4 : (live > 64 ? 2 : 1));
        // source row of each A row of the unit (rows past the expert's end repeat its last row)
        for (int r = threadIdx.x; r < kQBM; r += kQThreads) {
            int src = u.row0 + min(u.m0 + r, u.M - 1);
            if (p.gather) src = p.sorted_pairs[src] / p.k;
            s_arow[r] = min(max(src, 0), p.n_arows - 1);
        }
        __syncthreads();
        if (TM == 4) qgemm_unit<PAIR, 4, AS>(p, u, smem, s_arow);
        else if (TM == 2) qgemm_unit<PAIR, 2, AS>(p, u, smem, s_arow);
        else qgemm_unit<PAIR, 1, AS>(p, u, smem, s_arow);
        __syncthreads();                                     // the unit is done with s_arow and LDS
    }
}

// The matrix-core GEMM serves MX-quantised activations when there are enough rows per
// expert to fill its row tiles at least partly (prefill); decode sizes use the GEMV.
bool mfma_path_wanted(const moe_expert_weights *w, int act, int T, int k, bool routed) {
    (void)k;
    (void)routed;
    return act == MOE_ACT_MXFP4 && w->format == MOE_W_MXFP4 && T >= 64 && w->d_ff % 32 == 0 &&
           w->d_model % 32 == 0;
}

// Workgroups resident at once for a kernel on the current device (queried once per device).
template <bool PAIR, bool ROUTED, bool AS>
static int resident_workgroups() {
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mxgemm_kernel<PAIR, ROUTED, AS>, kQThreads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        cache[dev] = cus * per_cu;
    }
    return cache[dev];
}

// Persistent launch: at most one wave of resident workgroups, each walking the work units
// with a stride of the grid size.  `mt_bound` bounds the row tiles (4 parts each at most).
// The two-step scale windows need every scale row on a dword (K % 128 == 0, dword-aligned
// scale arrays) and at least two K-steps of scales per row (K >= 512).
template <bool PAIR, bool ROUTED>
static moe_status gemm_launch(const GemmParams &p, int mt_bound, hipStream_t stream, const char *what) {
    const int NB = PAIR ? kQBR / 2 : kQBR;
    const bool as = p.K % 128 == 0 && p.K >= 512 && ((uintptr_t)p.as & 3u) == 0 && ((uintptr_t)p.ws[0] & 3u) == 0 &&
                    (!PAIR || ((uintptr_t)p.ws[1] & 3u) == 0);
    const int64_t units = 4 * (int64_t)mt_bound * ((p.N + NB - 1) / NB);
    const int64_t g = std::min<int64_t>(units, as ? resident_workgroups<PAIR, ROUTED, true>()
                                                   : resident_workgroups<PAIR, ROUTED, false>());
    if (g <= 0) return MOE_OK;
    if (as)
        hipLaunchKernelGGL((mxgemm_kernel<PAIR, ROUTED, true>), dim3((unsigned)g), dim3(kQThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((mxgemm_kernel<PAIR, ROUTED, false>), dim3((unsigned)g), dim3(kQThreads), 0, stream, p);
    return launch_check(what);
}

static int tile_slots(const moe_expert_weights *w, int T, int R, bool routed) {
    if (!routed) return (T + kQBM - 1) / kQBM;
    const int ne = w->num_experts < R ? w->num_experts : R;
    return ne + R / kQBM;            // >= sum over experts of ceil(M_e / 256)
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

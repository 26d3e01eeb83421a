// Decode down product and weighted combine on the matrix cores, MXFP4 weights: the body of
// down_combine_mfma_kernel (gemv_mfma.hip) and of the down phase of decode_step_kernel
// (gemv.hip).
#pragma once

#include "gemv.h"
#include "step_sync.h"

namespace moe {

// ------------------------------------------------------------------ down + combine
// The decode down product with the weighted combine (as down_combine_kernel in gemv.hip),
// MXFP4 weights, multiply-adds on v_mfma_f32_16x16x32_bf16.
//
// The instruction's A operand puts row i of the tile in lanes i, 16 + i, 32 + i, 48 + i, so
// four neighbouring lanes hold four different rows; loaded in that layout, every group of
// four lanes reads from four weight rows, and the L1 handles each lane's 16 bytes as an
// access of its own.  Here four neighbouring lanes read four consecutive 16-byte units of
// one row instead: A row i = 4a + b is weight row a over part b, where part b of a step is
// the units 16m + 4g + b read by lane group g (g = 0..3).  B holds the slot's h in eight
// columns, column 2b + p being plane p (hi = RN_bf16(h), lo = RN_bf16(h - hi), together
// within 2^-17 |h|) at the units of part b; the other eight columns are zero.  Then
// C[4a + b][2b + p] is row a's dot product over part b with plane p, and the row's dot
// product is the sum of those eight entries.  A step covers 16 units (512 values) of 8 rows
// as two such tiles of 4 rows on one B: each load instruction reads 256 contiguous bytes of
// each of 4 rows, and each group of four lanes 64 of them.  The vector ALU only converts
// codes (one instruction per two weights) and advances pointers.
//
// Work items are (tile of 8 rows, slot j, K part kp): the item's rows of slot j over its
// part of the steps (two parts when an item has at least 2 * kDmDepth steps, else one).
// Waves take items from an LDS counter, so a wave that is served late takes fewer of them.
// Item (tile, j, kp) writes its 8 dot products to part[kp][j][rows] of an LDS table
// whatever wave ran it; after a barrier every row's output is the slot-ordered sum of
// w_j * (part[0] + part[1]), so the result does not depend on which wave ran what.  Each
// wave keeps kDmDepth steps of loads in flight across item boundaries; every slot of that
// ring records the position its loads belong to.
//
// Prologue: the slots' float32 h rows are loaded into registers first, then the weights of
// the wave's first two steps; the h values are written to LDS as the bf16 hi and lo planes
// slot by slot (each workgroup takes the slots in its own rotated order, so the CUs of a die
// do not all ask the L2 for the same lines at once, and its items follow the same order),
// and after each of its iterations a wave counts itself in that iteration's LDS counter.  An
// item waits only for the counter of the last iteration holding its slot's h, so the first
// slots' items start while the later slots' h is still arriving.  (A workgroup barrier
// there would also wait for the slowest wave to get its weight loads issued, and the waves
// already past it would issue nothing meanwhile.)
constexpr int kDmDepth = 4;              // steps of loads in flight per wave
constexpr int kDmThreads = 1024;         // 16 waves, four per SIMD
constexpr int kDmTile = 8;               // weight rows per item (two A tiles of 4 rows)
constexpr int kDmMaxGroups = 4800;       // 8-value groups of h: slots * dc_plane_ld(I) / 8 within 150 KiB
constexpr int kDmIters = (kDmMaxGroups + kDmThreads - 1) / kDmThreads;   // h groups per thread
static_assert(2 * kDmMaxRows <= kDcMaxRows, "two partial sums per row must fit the table");
static_assert(dc_plane_ld(1) % 512 == 0, "a plane must hold whole steps of 16 units");

static __device__ __align__(16) uint8_t g_dm_zero[16];   // read-only zeros (loads of a wave with no item left)

// STEP: the down phase of the single-launch decode step (decode_step_kernel): the slots'
// experts, rows and weights come from the workgroup's own routing in LDS, the weight loads
// of the ring's four steps are issued before the h rows are read (at device scope,
// step_get4), and with `wait_h` wave 0 first waits for every workgroup's h rows
// (step_wait) while those loads are in flight.
template <bool STEP>
MOE_DEV void dm_body(const DownCombineParams &p, int bx, int t, const StepCtx *sc, bool wait_h) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_e[MOE_MAX_TOPK + 1], s_r[MOE_MAX_TOPK + 1];
    __shared__ float s_w[MOE_MAX_TOPK + 1];
    __shared__ int s_item, s_ready[kDmIters];
    constexpr int NW = kDmThreads / 64;
    const int nslot = p.k + (p.sw ? 1 : 0);
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    if constexpr (STEP) __syncthreads();                   // the previous item's table reads are done
    if (tid < nslot) {
        int e = 0, r = t;
        float wt = p.sg ? (STEP ? sc->lds->sg[t] : p.sg[t]) : 1.0f;
        if (tid < p.k) {
            const int pi = t * p.k + tid;
            e = STEP ? sc->lds->ids[pi] : p.ids[pi];
            r = STEP ? sc->lds->p2r[pi] : p.p2r[pi];
            wt = STEP ? sc->lds->tw[pi] : p.tw[pi];
            if (e < 0 || e >= p.E || r < 0 || r >= p.R) {      // dropped pair: contributes 0
                e = r = -1;
                wt = 0.0f;
            }
        }
        s_e[tid] = e;
        s_r[tid] = r;
        s_w[tid] = wt;
    }
    if (tid == 0) {
        s_item = NW;
#pragma unroll
        for (int u = 0; u < kDmIters; ++u) s_ready[u] = 0;
    }
    __syncthreads();

    // parameters in locals: a lambda that captures the parameter block by reference keeps it
    // in scratch memory, and a select between two of its fields becomes a select of addresses
    const int I = p.I, N = p.N, kk = p.k, rpw = p.rows_per_wg;
    const uint8_t *w_r = p.w, *w_s = p.sw;
    const uint8_t *s_rt = (const uint8_t *)p.s, *s_s = (const uint8_t *)p.ss;
    const int units = I / 32;
    const int nm = (units + 15) / 16;                      // steps per (tile, slot)
    const int ld = dc_plane_ld(p.I);                       // bf16 values per plane (>= 512 * nm)
    const int n_begin = bx * p.rows_per_wg;
    const int n_end = min(p.N, n_begin + p.rows_per_wg);
    if (n_begin >= n_end) return;                          // the whole workgroup (uniform)
    const int ntile = (n_end - n_begin + kDmTile - 1) / kDmTile;
    const int KS = nm >= 2 * kDmDepth ? 2 : 1;             // K parts per (tile, slot)
    const int per_pos = ntile * KS;                        // items per slot position
    const int nitems = nslot * per_pos;
    // slot order of this workgroup: position q is slot (q + srot) mod nslot, for the items and
    // for the h rows alike, so that the CUs of a die do not all read the same h lines first
    const int srot = (int)(((long long)bx * 5 + (long long)t * 3) % nslot);
    const int per = ld / 8;                                // 8-value groups of h per slot
    const int i16 = lane & 15, g = lane >> 4;
    const int ra = i16 >> 2, pb = i16 & 3;                 // A: row ra (+ 4) of the tile, part pb
    uint16_t *planes = (uint16_t *)smem;                   // slot j: hi plane 2j, lo plane 2j+1
    float *part = (float *)(smem + p.h_lds_bytes);          // [2][nslot][rows_per_wg]
    const uint32_t row_bytes = (uint32_t)I / 2;

    // load cursor: item `it` (nitems: none left), step m of [m, m_end); matrix bases of the
    // item (wave-uniform) and this lane's offsets of its two rows
    int it = min(wave, nitems), m = 0, m_end = 0, cj = 0, ctile = 0, ckp = 0, cpos = 0;
    const uint8_t *cwb = g_dm_zero, *csb = g_dm_zero;
    uint32_t cwo0 = 0, cwo1 = 0, cso0 = 0, cso1 = 0;
    auto setup = [&]() __attribute__((always_inline)) {     // (branch-free: a wave with no item left reads zeros)
        const bool has = it < nitems;
        const int itc = has ? it : 0;
        cpos = itc / per_pos;                              // items are slot-position major
        const int rem = itc - cpos * per_pos;
        ctile = rem / KS;
        ckp = rem - ctile * KS;
        cj = cpos + srot >= nslot ? cpos + srot - nslot : cpos + srot;
        m = has ? ckp * nm / KS : 0;
        m_end = has ? (ckp + 1) * nm / KS : 0;
        const bool sh = cj >= kk;
        const int e = max(__builtin_amdgcn_readfirstlane(s_e[cj]), 0);   // (the shared slot's entry is 0)
        const size_t first_row = (size_t)e * N;
        // (casts make both arms values: a conditional on two captured variables is an lvalue,
        // compiled as a select of their addresses, which keeps them in scratch memory)
        const uint8_t *wbase = sh ? (const uint8_t *)w_s : (const uint8_t *)w_r;
        const uint8_t *sbase = sh ? (const uint8_t *)s_s : (const uint8_t *)s_rt;
        cwb = has ? wbase + first_row * row_bytes : g_dm_zero;
        csb = has ? sbase + first_row * units : g_dm_zero;
        // rows past the range repeat its last row (their results are not stored)
        const uint32_t n0 = (uint32_t)min(n_begin + ctile * kDmTile + ra, n_end - 1);
        const uint32_t n1 = (uint32_t)min(n_begin + ctile * kDmTile + 4 + ra, n_end - 1);
        cwo0 = has ? n0 * row_bytes : 0u;
        cwo1 = has ? n1 * row_bytes : 0u;
        cso0 = has ? n0 * (uint32_t)units : 0u;
        cso1 = has ? n1 * (uint32_t)units : 0u;
    };
    auto grab = [&]() __attribute__((always_inline)) {
        int v = 0;
        if (lane == 0) v = atomicAdd(&s_item, 1);
        return min(__builtin_amdgcn_readfirstlane(v), nitems);
    };
    // Loads are issued unconditionally (a load under a branch leaves the compiler unable
    // to count the loads in flight, and it then waits for all of them); a wave with no item
    // left reads a 16-byte block of zeros that stays in cache.  Units past the row repeat
    // its last unit (their scale is taken as 0 when converted).
    auto load = [&](u32x4 (&w)[2], uint8_t (&sc)[2]) __attribute__((always_inline)) {
        const bool lv = it < nitems;
        const uint32_t u = (uint32_t)min(16 * m + 4 * g + pb, units - 1);
        w[0] = *(const u32x4 *)(cwb + (lv ? cwo0 + u * 16 : 0u));
        w[1] = *(const u32x4 *)(cwb + (lv ? cwo1 + u * 16 : 0u));
        sc[0] = csb[lv ? cso0 + u : 0u];
        sc[1] = csb[lv ? cso1 + u : 0u];
    };
    // ring slot d: the position its loads belong to
    int pj[kDmDepth], ptile[kDmDepth], pkp[kDmDepth], pm[kDmDepth], ppos[kDmDepth];
    bool plive[kDmDepth], plast[kDmDepth];
    int live_slots = 0;
    auto fill = [&](auto dc, u32x4 (&w)[2], uint8_t (&sc)[2]) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        const bool lv = it < nitems;
        pj[d] = cj;
        ppos[d] = cpos;
        ptile[d] = ctile;
        pkp[d] = ckp;
        pm[d] = m;
        plive[d] = lv;
        plast[d] = m + 1 == m_end;
        load(w, sc);
        live_slots += lv ? 1 : 0;
        if (lv && ++m == m_end) {
            it = grab();
            setup();
        }
    };

    f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    u32x4 bq[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};   // zero outside columns 0..7
    // Step of ring slot d into acc (units past the row get scale 0, so A is zero there, and
    // the planes are zero past d_ff); the item's last step sums each row's eight entries and
    // stores the tile's 8 dot products (0 for a dropped pair).
    auto compute = [&](auto dc, const u32x4 (&w)[2], const uint8_t (&sc)[2]) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        const int j = pj[d];
        // B lane (column i16 < 8, group g): plane i16 & 1 of slot j at unit 16m + 4g + i16 / 2
        const uint16_t *bp = planes + (size_t)(2 * j + (i16 & 1)) * ld + (16 * pm[d] + 4 * g + (i16 >> 1)) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (i16 < 8) bq[q] = *(const u32x4 *)(bp + 8 * q);
        const bool uin = 16 * pm[d] + 4 * g + pb < units;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 a[4];
            unit_to_bf16x8(w[h], uin ? e8m0_to_f32(sc[h]) : 0.0f, a);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], __builtin_bit_cast(bf16x8, bq[q]), acc[h], 0, 0, 0);
        }
        if (!plast[d]) return;
        const bool drop = __builtin_amdgcn_readfirstlane(s_e[j]) < 0;
        float *pp = part + (size_t)(pkp[d] * nslot + j) * rpw;
        // lane (column c = i16, group G = g) holds C[4G + v][c]: row G of the A tile over part
        // v; the entries of row G are those with c < 8, v = c / 2
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int v = i16 >> 1;
            float x = v == 0 ? acc[h][0] : v == 1 ? acc[h][1] : v == 2 ? acc[h][2] : acc[h][3];
            x = i16 < 8 ? x : 0.0f;
            x += __shfl_xor(x, 1, kWave);
            x += __shfl_xor(x, 2, kWave);
            x += __shfl_xor(x, 4, kWave);
            if (drop) x = 0.0f;
            const int lr = ptile[d] * kDmTile + 4 * h + g;
            if (i16 == 0 && n_begin + lr < n_end) pp[lr] = x;
            acc[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    // h rows -> registers: 8-value group i = (slot j, group v) of the planes' layout, taken
    // from a workgroup-dependent starting point; groups past d_ff and dropped slots become
    // zeros when written (their loads read a valid group).
    constexpr int kGroups = kDmIters;
    const int total = nslot * per;
    auto group_of = [&](int i) __attribute__((always_inline)) {   // linear index -> group (slot order)
        const int r = i + srot * per;
        return r >= total ? r - total : r;
    };
    f32x4 va[kGroups], vb[kGroups];
    auto load_h = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
            const int i = group_of(min(tid + u * kDmThreads, total - 1));
            const int j = i / per, v = min(i - j * per, I / 8 - 1);
            const float *row = j < kk ? p.h + (size_t)max(s_r[j], 0) * I : p.hs + (size_t)t * I;
            if constexpr (STEP) {
                va[u] = step_get4(row + (size_t)v * 8);
                vb[u] = step_get4(row + (size_t)v * 8 + 4);
            } else {
                const f32x4 *src = (const f32x4 *)(row + (size_t)v * 8);
                va[u] = src[0];
                vb[u] = src[1];
            }
        }
    };
    u32x4 wv[kDmDepth][2];
    uint8_t sv[kDmDepth][2];  // (the loaded bytes as they are: a value combined from two loads waits for both)
    static_assert(kDmDepth == 4, "the prologue issues two steps before the planes and two after");
    if constexpr (STEP) {
        // the weights do not depend on h: the ring's loads go out before the wait
        setup();
        fill(std::integral_constant<int, 0>{}, wv[0], sv[0]);
        fill(std::integral_constant<int, 1>{}, wv[1], sv[1]);
        fill(std::integral_constant<int, 2>{}, wv[2], sv[2]);
        fill(std::integral_constant<int, 3>{}, wv[3], sv[3]);
        if (wait_h) {
            if (wave == 0) step_wait(sc->sync, sc->nwg, sc->tag);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        load_h();
    } else {
        load_h();
        setup();
        fill(std::integral_constant<int, 0>{}, wv[0], sv[0]);
        fill(std::integral_constant<int, 1>{}, wv[1], sv[1]);
    }
    // float32 h -> bf16 hi/lo planes: hi = RN_bf16(h), lo = RN_bf16(h - hi) by the packed
    // round-to-nearest-even conversion; plane hi of slot j at element 2j*ld, lo at (2j+1)*ld.
    // Iteration u covers linear indices [1024u, 1024(u+1)), i.e. slot positions in order; each
    // wave counts itself in s_ready[u] after its writes of iteration u, so the items of a slot
    // position can start once every wave is past the last iteration holding its groups.
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
        if (tid + u * kDmThreads < total) {
        const int i = group_of(tid + u * kDmThreads);
        const int j = i / per, v = i - j * per;
        const bool ok = v * 8 < I && (j >= kk || s_r[j] >= 0);
        const f32x4 x0 = ok ? va[u] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const f32x4 x1 = ok ? vb[u] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const f32x2 f[4] = {{x0[0], x0[1]}, {x0[2], x0[3]}, {x1[0], x1[1]}, {x1[2], x1[3]}};
        u32x4 hv, lv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f[q], bf16x2));
            const f32x2 r = {f[q].x - __uint_as_float(hb << 16), f[q].y - __uint_as_float(hb & 0xffff0000u)};
            hv[q] = hb;
            lv[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        }
        *(u32x4 *)(planes + (size_t)(2 * j) * ld + v * 8) = hv;
        *(u32x4 *)(planes + (size_t)(2 * j + 1) * ld + v * 8) = lv;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's writes of iteration u are in LDS
        if (lane == 0) atomicAdd(&s_ready[u], 1);
    }
    if constexpr (!STEP) {
        fill(std::integral_constant<int, 2>{}, wv[2], sv[2]);
        fill(std::integral_constant<int, 3>{}, wv[3], sv[3]);
    }
    // Before an item's steps: wait until every wave has written the planes of its slot
    // position (a wave's positions only increase).  Every wave counts itself in each counter,
    // right after its writes, so the wait ends; the bound only keeps a fault elsewhere from
    // turning into a hang.  (Read through an LDS pointer: a generic volatile read is a flat
    // load, and its wait would also wait for every weight load in flight.)
    int ready_known = -1;
    auto wait_planes = [&](int pos) __attribute__((always_inline)) {
        const int need = ((pos + 1) * per - 1) / kDmThreads;
        if (need <= ready_known) return;
        volatile __attribute__((address_space(3))) int *ready =
            (volatile __attribute__((address_space(3))) int *)&s_ready[need];
        for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__builtin_amdgcn_readfirstlane(*ready) >= NW) break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");                     // no plane read moves above the wait
        ready_known = need;
    };

    while (live_slots > 0) {
        static_for<kDmDepth>([&](auto dc) __attribute__((always_inline)) {
            constexpr int d = decltype(dc)::value;
            if (plive[d]) {
                wait_planes(ppos[d]);
                compute(dc, wv[d], sv[d]);
                --live_slots;
            }
            fill(dc, wv[d], sv[d]);
        });
    }
    __syncthreads();
    const float *q0p = part, *q1p = part + (size_t)nslot * p.rows_per_wg;
    for (int lr = tid; lr < n_end - n_begin; lr += kDmThreads) {
        float o = 0.0f;
        for (int j = 0; j < nslot; ++j) {                  // slot order
            const float v = KS == 2 ? q0p[j * p.rows_per_wg + lr] + q1p[j * p.rows_per_wg + lr]
                                    : q0p[j * p.rows_per_wg + lr];
            o = fmaf(s_w[j], v, o);
        }
        p.out[(size_t)t * p.N + n_begin + lr] = o;
    }
}

}  // namespace moe

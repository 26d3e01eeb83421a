// Decode down product and weighted combine on the matrix cores, MXFP4 weights.
#include "gemv.h"

namespace moe {

// ------------------------------------------------------------------ down + combine
// The decode down product with the weighted combine (as down_combine_kernel in gemv.hip),
// MXFP4 weights, multiply-adds on v_mfma_f32_16x16x32_bf16.  A wave's work item is a tile
// of 16 weight rows of one slot.  A step covers one 128-byte line of each row (8 units,
// 256 values) as two K-steps of 128: lane l loads units 8m + l/16 and 8m + 4 + l/16 of row
// l%16 and converts each to its A slices for four MFMAs.  B holds the slot's h as two bf16
// columns, hi = RN_bf16(h) and lo = RN_bf16(h - hi) (together within 2^-17 |h|), the other
// 14 columns zero, so C[row][0] + C[row][1] is the row's dot product.  The vector ALU only
// converts codes (one instruction per two weights) and advances pointers: the float32
// multiply-adds of the vector kernel cost as much issue time as the HBM stream.  Each wave
// keeps kDmDepth steps of loads in flight across item boundaries; results go through the
// part[slot][row] LDS table and the slot-ordered final sum.
#ifndef MOE_DM_DEPTH
#define MOE_DM_DEPTH 4           // steps of loads in flight per wave
#endif
#ifndef MOE_DM_NT
#define MOE_DM_NT 0              // non-temporal weight loads (off: the two half-lines of a row arrive in separate loads)
#endif
constexpr int kDmDepth = MOE_DM_DEPTH;

MOE_DEV void dm_dma16(const void *src, uint32_t lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

__device__ __align__(16) uint8_t g_dm_zero[16];   // read-only zeros (loads past a wave's work)

// A wave's position: step m of item (tile, slot j), with the item's matrix bases
// (wave-uniform) and this lane's row offsets.
struct DmIt {
    int q, j, m, tile;
    const uint8_t *wb, *sb;
    uint32_t wo, so;
};

#ifndef MOE_DM_THREADS
#define MOE_DM_THREADS 1024      // threads of a matrix-core down-combine workgroup (4 waves per SIMD)
#endif
constexpr int kDmThreads = MOE_DM_THREADS;

__global__ __launch_bounds__(kDmThreads) void down_combine_mfma_kernel(const DownCombineParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_e[MOE_MAX_TOPK + 1], s_r[MOE_MAX_TOPK + 1];
    __shared__ float s_w[MOE_MAX_TOPK + 1];
    constexpr int NW = kDmThreads / 64;
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

    const int units = p.I / 32;
    const int nm = (units + 7) / 8;                        // steps per item
    const int ld = dc_plane_ld(p.I);                       // bf16 values per plane (>= 256 * nm)
    const int n_begin = blockIdx.x * p.rows_per_wg;
    const int n_end = min(p.N, n_begin + p.rows_per_wg);
    if (n_begin >= n_end) return;                          // the whole workgroup
    const int ntile = (n_end - n_begin + 15) / 16;
    const int nitems = ntile * nslot;
    const int my_items = wave < nitems ? (nitems - 1 - wave) / NW + 1 : 0;
    const int nq = my_items * nm;
    const int r16 = lane & 15, g = lane >> 4;
    uint16_t *planes = (uint16_t *)smem;                   // slot j: hi plane 2j, lo plane 2j+1
    float *part = (float *)(smem + p.h_lds_bytes);          // [nslot][rows_per_wg]
    const uint32_t row_bytes = (uint32_t)p.I / 2;

    auto setup = [&](DmIt &c) {
        const bool sh = c.j >= p.k;
        const int e = sh ? 0 : max(__builtin_amdgcn_readfirstlane(s_e[c.j]), 0);
        const size_t first_row = (size_t)e * p.N;
        c.wb = (sh ? p.sw : p.w) + first_row * row_bytes;
        c.sb = (const uint8_t *)(sh ? p.ss : p.s) + first_row * units;
        const uint32_t n = (uint32_t)min(n_begin + c.tile * 16 + r16, n_end - 1);
        c.wo = n * row_bytes;
        c.so = n * (uint32_t)units;
    };
    auto advance = [&](DmIt &c) {
        ++c.q;
        if (++c.m == nm) {
            c.m = 0;
            c.j += NW;
            while (c.j >= nslot) {
                c.j -= nslot;
                ++c.tile;
            }
            setup(c);
        }
    };
    // Loads are issued unconditionally (a load under a branch leaves the compiler unable
    // to count the loads in flight, and it then waits for all of them); positions past the
    // wave's last step read a 16-byte block of zeros that stays in cache.
    auto load = [&](const DmIt &c, u32x4 (&w)[2], uint8_t (&sc)[2]) {
        const bool live = c.q < nq;
        const uint8_t *wb = live ? c.wb : g_dm_zero;
        const uint8_t *sb = live ? c.sb : g_dm_zero;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t u = (uint32_t)min(8 * c.m + 4 * h + g, units - 1);
            const u32x4 *src = (const u32x4 *)(wb + (live ? c.wo + u * 16 : 0u));
            if constexpr (MOE_DM_NT) w[h] = __builtin_nontemporal_load(src);
            else w[h] = *src;
            sc[h] = sb[live ? c.so + u : 0u];
        }
    };
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 bq[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};   // zero outside columns 0, 1
    // Step at c into acc (units past the row get scale 0, so A is zero there, and B is zero
    // past d_ff); the item's last step adds the hi and lo columns and stores the tile's 16
    // dot products for slot j (0 for a dropped pair).
    auto compute = [&](const DmIt &c, const u32x4 (&w)[2], const uint8_t (&sc)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int u = 8 * c.m + 4 * h + g;
            bf16x8 a[4];
            unit_to_bf16x8(w[h], u < units ? e8m0_to_f32((uint32_t)sc[h]) : 0.0f, a);
            const uint16_t *bp = planes + (size_t)(2 * c.j + (r16 & 1)) * ld + u * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (r16 < 2) bq[q] = *(const u32x4 *)(bp + 8 * q);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], __builtin_bit_cast(bf16x8, bq[q]), acc, 0, 0, 0);
            }
        }
        if (c.m != nm - 1) return;
        const bool drop = __builtin_amdgcn_readfirstlane(s_e[c.j]) < 0;
        // lane (col r16, group g) holds C[4g+v][r16]; column 1 moves down one lane
        const int l0 = c.tile * 16 + 4 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float o = acc[v] + __shfl_down(acc[v], 1, kWave);
            if (drop) o = 0.0f;
            if (r16 == 0 && n_begin + l0 + v < n_end) part[c.j * p.rows_per_wg + l0 + v] = o;
            acc[v] = 0.0f;
        }
    };

    // h rows -> LDS by direct copies: slot j's float32 row at byte 4*ld*j, in whole 1 KiB
    // blocks (the tail of a row's last block re-reads its last vector into the row's
    // padding; 4*ld is a multiple of 1 KiB).  The copies are waited for before any weight
    // load is issued: behind a full pipeline of weight loads they would land several times
    // later.  The first kDmDepth steps of weight loads are then in flight during the
    // conversion, whose barriers wait for LDS accesses only (a __syncthreads would also wait
    // for every load in flight).
    {
        const int act_vec = p.I / 4;
        const int bpr = (act_vec + 63) / 64;                 // copy blocks per row
        for (int blk = wave; blk < nslot * bpr; blk += NW) {
            const int j = blk / bpr, b0 = (blk - j * bpr) * 64;
            const int v = min(b0 + lane, act_vec - 1);
            const float *row = j < p.k ? p.h + (size_t)max(s_r[j], 0) * p.I : p.hs + (size_t)t * p.I;
            dm_dma16(row + (size_t)v * 4, (uint32_t)(uintptr_t)(smem + (size_t)j * 4 * ld + (size_t)b0 * 16));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    u32x4 wv[kDmDepth][2];
    uint8_t sv[kDmDepth][2];  // (bytes: a widened copy would be masked at the loop latch, forcing a wait)
    DmIt lp{0, wave % nslot, 0, wave / nslot, nullptr, nullptr, 0, 0};
    setup(lp);
    const DmIt first = lp;
#pragma unroll
    for (int d = 0; d < kDmDepth; ++d) {
        load(lp, wv[d], sv[d]);
        advance(lp);
    }
    // float32 rows -> bf16 hi/lo planes in place (all reads before the barrier, all writes
    // after): plane hi at element 0 of the row's region, lo at element ld; zeros past d_ff
    // and for dropped pairs.  hi = RN_bf16(h), lo = RN_bf16(h - hi) by the packed
    // round-to-nearest-even conversion.
    {
        // 8-value groups: S * ld / 8 in all, S * 4 * ld <= 150 KiB -> <= 4800
        constexpr int kGroups = (4800 + kDmThreads - 1) / kDmThreads;
        const int per = ld / 8;
        const int total = nslot * per;
        f32x4 va[kGroups], vb[kGroups];
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
            const int i = min(tid + u * kDmThreads, total - 1);
            const int j = i / per, v = i - j * per;
            const bool ok = v * 8 < p.I && (j >= p.k || s_r[j] >= 0);
            const f32x4 *src = (const f32x4 *)(smem + (size_t)j * 4 * ld) + 2 * v;
            va[u] = ok ? src[0] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            vb[u] = ok ? src[1] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
            const int i = tid + u * kDmThreads;
            if (i >= total) break;
            const int j = i / per, v = i - j * per;
            const f32x2 f[4] = {{va[u][0], va[u][1]}, {va[u][2], va[u][3]}, {vb[u][0], vb[u][1]}, {vb[u][2], vb[u][3]}};
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
    }
    lds_barrier();

    DmIt cp = first;
    for (int q0 = 0; q0 < nq; q0 += kDmDepth) {
#pragma unroll
        for (int d = 0; d < kDmDepth; ++d) {
            if (cp.q < nq) compute(cp, wv[d], sv[d]);
            advance(cp);
            load(lp, wv[d], sv[d]);
            advance(lp);
        }
    }
    __syncthreads();
    for (int lr = tid; lr < n_end - n_begin; lr += kDmThreads) {
        float o = 0.0f;
        for (int j = 0; j < nslot; ++j) o = fmaf(s_w[j], part[j * p.rows_per_wg + lr], o);   // slot order
        p.out[(size_t)t * p.N + n_begin + lr] = o;
    }
}

void down_combine_mfma_launch(const DownCombineParams &p, dim3 grid, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL(down_combine_mfma_kernel, grid, dim3(kDmThreads), lds, stream, p);
}

}  // namespace moe

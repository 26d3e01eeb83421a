// Row-tile bookkeeping shared by the prefill grouped GEMMs.
//
// expert_offsets[e] .. expert_offsets[e+1] are the sorted rows routed to expert e.  A
// grouped GEMM covers each expert's rows with BM-row tiles; the tiles of all experts are
// numbered expert by expert, and every workgroup of a persistent grid rebuilds that
// numbering in LDS from the offsets instead of reading a host-built schedule.
#pragma once
#include "common.h"

namespace moe {

// Inclusive prefix over experts of their BM-row tile counts: tp[e] = tiles of experts
// 0..e (TP = int, or uint16_t where LDS is tight: R / BM + E < 65536).  Offsets outside
// [0, R] (or decreasing) give the expert no tiles.  Returns the total; every thread of the
// THREADS-wide workgroup must call it (it synchronises).
template <int THREADS, int BM, typename TP>
MOE_DEV int build_tile_prefix(const int32_t *offsets, int E, int R, TP *tp, int *s_wave) {
    constexpr int kPer = (MOE_MAX_EXPERTS + THREADS - 1) / THREADS;   // experts per thread
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    int t[kPer], sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = tid * kPer + u;
        const int lo = offsets[min(e, E)], hi = offsets[min(e + 1, E)];
        const int m = (e < E && lo >= 0 && hi <= R) ? max(hi - lo, 0) : 0;
        t[u] = (m + BM - 1) / BM;
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
    for (int w = 0; w < THREADS / 64; ++w) {
        base += w < wave ? s_wave[w] : 0;
        total += s_wave[w];
    }
    int run = base + incl - sum;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        run += t[u];
        const int e = tid * kPer + u;
        if (e < E) tp[e] = (TP)run;
    }
    __syncthreads();
    return total;
}

// Expert owning row tile mt: the first e with tp[e] > mt (E <= 64 * 32: two probes).
template <typename TP>
MOE_DEV int tile_expert(const TP *tp, int E, int mt) {
    const int lane = lane_id();
    const int probe = min(lane * 32 + 31, E - 1);
    const uint64_t m1 = __ballot(lane * 32 < E && (int)tp[probe] > mt);
    const int c = __ffsll((long long)m1) - 1;                  // chunk of 32 experts
    const int e2 = c * 32 + (lane & 31);
    const uint64_t m2 = __ballot(lane < 32 && e2 < E && (int)tp[min(e2, E - 1)] > mt);
    return c * 32 + __ffsll((long long)m2) - 1;
}

// Position of workgroup b in the item order: with G a multiple of 8, XCD x (workgroups
// x, x+8, ...) takes a contiguous run of G/8 items per round, so the row tiles of one expert
// that share a column tile of weights run together on one XCD and share its L2.
MOE_DEV int xcd_slot(int b, int G) { return (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b; }

static_assert(MOE_MAX_EXPERTS <= 64 * 32, "tile_expert probes at most 64 x 32 experts");

}  // namespace moe

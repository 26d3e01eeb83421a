// Token -> expert permutation: a stable counting sort of the T*k (token, slot) pairs.
//
// The pages group work per expert (rabbit README, features list: each expert's matmul
// starts when its own bytes land) and run a step's routed experts in one launch
// (Rulith Inference README, engine section).  Here: per-wave histograms of expert ids
// (LDS atomics -- counts do not depend on order), exclusive prefix scans giving each
// (wave, expert) its first row, and a scatter in which each wave places its pairs in
// order, ranking equal ids within a 64-pair chunk by wave ballots -- so positions never
// depend on timing.
#include "common.h"

namespace moe {
namespace {

constexpr int kPermWaves = 16;
constexpr int kPermThreads = 64 * kPermWaves;

// Lanes of the wave whose expert id equals this lane's (ids < 2^11; invalid lanes are in no
// set): the intersection, over the id's bits, of the lanes that agree on the bit.
MOE_DEV uint64_t lanes_with_same_id(int e, bool valid) {
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 11; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        m &= bit ? ones : ~ones;
    }
    return m;
}

// One workgroup.  Wave w owns a contiguous range of 64-pair chunks.  (1) Each wave counts
// its pairs per expert (LDS atomics: counts do not depend on order).  (2) A prefix over
// experts, then over waves, gives every (wave, expert) its first row.  (3) Each wave walks
// its chunks in order; a pair's row is its (wave, expert) base plus the number of lower
// lanes of the chunk with the same expert, and the group's lowest lane advances the base.
// Rows therefore follow the pair index within every expert, whatever the timing.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ ids, int P,
                                                               int E, int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ sorted,
                                                               int32_t *__restrict__ p2r) {
    extern __shared__ int wc[];            // [kPermWaves][E]: counts, then bases
    __shared__ int s_wave_tot[kPermWaves];
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wc[i] = 0;
    __syncthreads();
    const int nch = (P + 63) / 64;
    const int cpw = (nch + kPermWaves - 1) / kPermWaves;
    const int c0 = min(nch, wave * cpw), c1 = min(nch, c0 + cpw);
    int *mine = wc + wave * E;
    for (int c = c0; c < c1; ++c) {
        const int p = c * 64 + lane;
        const int e = p < P ? ids[p] : -1;
        if (e >= 0 && e < E) atomicAdd(&mine[e], 1);
    }
    __syncthreads();

    // (2) totals per expert, exclusive scan over experts (E <= 2 * kPermThreads: two per
    // thread), then bases per wave
    const int ea = 2 * tid, eb = 2 * tid + 1;
    int ta = 0, tb = 0;
    if (ea < E)
        for (int w = 0; w < kPermWaves; ++w) ta += wc[w * E + ea];
    if (eb < E)
        for (int w = 0; w < kPermWaves; ++w) tb += wc[w * E + eb];
    int incl = ta + tb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kPermWaves; ++w) {
        if (w < wave) base += s_wave_tot[w];
        total += s_wave_tot[w];
    }
    int oa = base + incl - (ta + tb), ob = oa + ta;
    if (ea < E) offsets[ea] = oa;
    if (eb < E) offsets[eb] = ob;
    if (tid == 0) offsets[E] = total;
    if (ea < E)
        for (int w = 0; w < kPermWaves; ++w) {
            const int c = wc[w * E + ea];
            wc[w * E + ea] = oa;
            oa += c;
        }
    if (eb < E)
        for (int w = 0; w < kPermWaves; ++w) {
            const int c = wc[w * E + eb];
            wc[w * E + eb] = ob;
            ob += c;
        }
    for (int r = total + tid; r < P; r += kPermThreads) sorted[r] = -1;
    __syncthreads();

    // (3) stable scatter, chunk by chunk
    const uint64_t below = (1ull << lane) - 1ull;
    for (int c = c0; c < c1; ++c) {
        const int p = c * 64 + lane;
        const int e = p < P ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        const uint64_t same = lanes_with_same_id(e, valid);
        if (valid) {
            const int r = mine[e] + __popcll(same & below);
            sorted[r] = p;
            p2r[p] = r;
        } else if (p < P) {
            p2r[p] = -1;
        }
        // the group's lowest lane moves the base past the group (after every lane read it:
        // a wave's LDS accesses complete in order)
        if (valid && (same & below) == 0) mine[e] += __popcll(same);
    }
}

// Few pairs (decode): P <= 64, ranks by counting (small_permutation).  Same results as
// the counting sort, one barrier, no scan.
constexpr int kPermSmallP = 64;

__global__ __launch_bounds__(256) void permute_small_kernel(const int32_t *__restrict__ ids, int P, int E,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted,
                                                            int32_t *__restrict__ p2r) {
    __shared__ int sid[kPermSmallP];
    const int tid = threadIdx.x;
    if (tid < kPermSmallP) {
        int e = tid < P ? ids[tid] : -1;
        sid[tid] = (e >= 0 && e < E) ? e : -1;
    }
    __syncthreads();
    small_permutation(sid, P, E, offsets, sorted, p2r, tid, blockDim.x);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace(int32_t, int32_t, int32_t) { return 0; }

extern "C" moe_status moe_permute(int32_t T, int32_t k, int32_t E, const int32_t *topk_ids,
                                  int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_to_row,
                                  void *, size_t, moe_stream stream) {
    clear_error();
    MOE_REQUIRE(T >= 0, "moe_permute: T = %d < 0", T);
    MOE_REQUIRE(E >= 1 && E <= MOE_MAX_EXPERTS, "moe_permute: E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
    MOE_REQUIRE(k >= 1 && k <= MOE_MAX_TOPK && k <= E, "moe_permute: k = %d outside [1, min(E, %d)]", k,
                MOE_MAX_TOPK);
    MOE_REQUIRE((int64_t)T * k < INT32_MAX, "moe_permute: T*k overflows int32");
    MOE_REQUIRE(expert_offsets != nullptr, "moe_permute: NULL expert_offsets");
    if (T > 0) MOE_REQUIRE(topk_ids && sorted_pairs && pair_to_row, "moe_permute: NULL pointer argument");
    const int P = T * k;
    if (P <= kPermSmallP) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, topk_ids, P, E,
                           expert_offsets, sorted_pairs, pair_to_row);
        return launch_check("moe_permute: permute_small_kernel");
    }
    const size_t lds = (size_t)kPermWaves * E * sizeof(int);
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, (hipStream_t)stream, topk_ids, P, E,
                       expert_offsets, sorted_pairs, pair_to_row);
    return launch_check("moe_permute: permute_kernel");
}

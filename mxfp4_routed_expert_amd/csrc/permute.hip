// Token -> expert permutation: a stable counting sort of the T*k (token, slot) pairs.
//
// The pages group work per expert (rabbit README, features list: each expert's matmul
// starts when its own bytes land) and run a step's routed experts in one launch
// (Rulith Inference README, engine section).  Here: a histogram of expert ids (LDS
// atomics -- counts do not depend on order), an exclusive prefix scan giving each
// expert's first row, and a stable scatter in which every expert walks the pairs in
// ascending order, so positions never depend on timing.
#include "common.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermIdCache = 12288;   // pair ids cached in LDS when P fits

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ ids, int P,
                                                               int E, int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ sorted,
                                                               int32_t *__restrict__ p2r) {
    extern __shared__ int smem[];
    int *cnt = smem;                       // [E + 1]
    int *sid = smem + E + 1;               // [P] when cached
    __shared__ int s_wave_tot[kPermThreads / 64];
    const bool cached = P <= kPermIdCache;
    const int tid = threadIdx.x;

    for (int i = tid; i <= E; i += kPermThreads) cnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kPermThreads) {
        const int e = ids[p];
        if (cached) sid[p] = e;
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
        else p2r[p] = -1;
    }
    __syncthreads();

    // exclusive scan of cnt[0..E) -> cnt (E <= 2 * kPermThreads): each thread owns two
    // consecutive counts; wave-level inclusive scan of pair sums, then wave totals.
    const int a0 = 2 * tid < E ? cnt[2 * tid] : 0;
    const int a1 = 2 * tid + 1 < E ? cnt[2 * tid + 1] : 0;
    int incl = a0 + a1;
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_wave_tot[wave_id()] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kPermThreads / 64; ++w) {
        if (w < wave_id()) base += s_wave_tot[w];
        total += s_wave_tot[w];
    }
    const int excl = base + incl - (a0 + a1);
    if (2 * tid < E) cnt[2 * tid] = excl;
    if (2 * tid + 1 < E) cnt[2 * tid + 1] = excl + a0;
    if (tid == 0) cnt[E] = total;
    __syncthreads();
    for (int e = tid; e <= E; e += kPermThreads) offsets[e] = cnt[e];
    for (int r = total + tid; r < P; r += kPermThreads) sorted[r] = -1;

    // stable scatter: expert e visits the pairs in ascending order.
    for (int e = tid; e < E; e += kPermThreads) {
        int r = cnt[e];
        const int end = cnt[e + 1];
        if (r == end) continue;
        for (int p = 0; p < P && r < end; ++p) {
            const int id = cached ? sid[p] : ids[p];
            if (id == e) {
                sorted[r] = p;
                p2r[p] = r;
                ++r;
            }
        }
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

// Many pairs (prefill): a bitonic sort of the unique keys (expert << s) | p in LDS by one
// workgroup gives the stable order directly, whatever the routing skew; invalid ids sort
// last.  Offsets come from the same histogram + scan as the counting sort.
constexpr int kPermSortMax = 8192;

__global__ __launch_bounds__(1024) void permute_sort_kernel(const int32_t *__restrict__ ids, int P, int E, int n2,
                                                            int shift, int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted,
                                                            int32_t *__restrict__ p2r) {
    extern __shared__ uint32_t keys[];          // [n2]
    __shared__ int cnt[MOE_MAX_EXPERTS + 1];
    __shared__ int s_wave_tot[16];
    const int tid = threadIdx.x;
    for (int i = tid; i <= E; i += 1024) cnt[i] = 0;
    __syncthreads();
    for (int i = tid; i < n2; i += 1024) {
        uint32_t key = 0xffffffffu;
        if (i < P) {
            const int e = ids[i];
            if (e >= 0 && e < E) {
                key = ((uint32_t)e << shift) | (uint32_t)i;
                atomicAdd(&cnt[e], 1);
            } else {
                p2r[i] = -1;
            }
        }
        keys[i] = key;
    }
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n2; i += 1024) {
                const int l = i ^ j;
                if (l > i) {
                    const uint32_t a = keys[i], b = keys[l];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        keys[i] = b;
                        keys[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    // exclusive scan of the counts (E <= 2048: two per thread)
    const int a0 = 2 * tid < E ? cnt[2 * tid] : 0;
    const int a1 = 2 * tid + 1 < E ? cnt[2 * tid + 1] : 0;
    int incl = a0 + a1;
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_wave_tot[wave_id()] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave_id()) base += s_wave_tot[w];
        total += s_wave_tot[w];
    }
    const int excl = base + incl - (a0 + a1);
    if (2 * tid < E) offsets[2 * tid] = excl;
    if (2 * tid + 1 < E) offsets[2 * tid + 1] = excl + a0;
    if (tid == 0) offsets[E] = total;
    const uint32_t pmask = (1u << shift) - 1u;
    for (int r = tid; r < P; r += 1024) {
        if (r < total) {
            const int pp = (int)(keys[r] & pmask);
            sorted[r] = pp;
            p2r[pp] = r;
        } else {
            sorted[r] = -1;
        }
    }
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
    if (P <= kPermSortMax) {
        int n2 = 1, shift = 0;
        while (n2 < P) n2 <<= 1;
        while ((1 << shift) < P) ++shift;
        hipLaunchKernelGGL(permute_sort_kernel, dim3(1), dim3(1024), (size_t)n2 * sizeof(uint32_t), (hipStream_t)stream,
                           topk_ids, P, E, n2, shift, expert_offsets, sorted_pairs, pair_to_row);
        return launch_check("moe_permute: permute_sort_kernel");
    }
    const size_t lds = (size_t)(E + 1 + (P <= kPermIdCache ? P : 0)) * sizeof(int);
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), lds, (hipStream_t)stream, topk_ids, P, E,
                       expert_offsets, sorted_pairs, pair_to_row);
    return launch_check("moe_permute: permute_kernel");
}

// Router: logits, scoring, top-k and renormalisation.
//
// Routing schemes of the pages: "softmax top-10 of 512 + gated shared expert"
// (Qwen3.8-Max) and "noaux_tc sigmoid" (GLM-5.2) -- rabbit README, architecture table,
// "MoE routing" row.  The logit of (t, e) is the float32 rounding of the exact dot
// product of two bf16 vectors: bf16 x bf16 products are exact in float64 and the sum
// is accumulated in float64, then rounded once.  Scoring, top-k and the weights run in
// float64; only the final weights are rounded to float32.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <mutex>

#include "common.h"

namespace moe {
namespace {

constexpr int kRouterTB = 8;      // tokens per wave
constexpr int kRouterUnroll = 4;  // 16-byte loads in flight per lane per pass

// A workgroup computes the dot products of one weight row (expert e < E, or the shared
// gate row e == E) with up to kRouterTB tokens; wave w covers the w-th quarter of H, so a
// row is read with four waves' worth of loads in flight.  Lanes stride over the quarter in
// 8-element (16-byte) vectors; loads are issued unconditionally from clamped indices (a
// load under a branch would be waited for at the join) and out-of-range vectors are
// skipped when consumed.  Float64 partial sums are reduced over the wave in a fixed
// butterfly order, then over the four waves in order.
constexpr int kRouterWaves = 4;

__global__ __launch_bounds__(64 * kRouterWaves) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                                         const uint16_t *__restrict__ wr,
                                                                         const uint16_t *__restrict__ wsg,
                                                                         int T, int H, int E, int rows,
                                                                         float *__restrict__ logits) {
    __shared__ double part[kRouterWaves][kRouterTB];
    const int row = blockIdx.x;
    const uint16_t *w = row < E ? wr + (size_t)row * H : wsg;
    const int t0 = blockIdx.y * kRouterTB;
    const int nt = min(kRouterTB, T - t0);
    const int lane = lane_id(), wave = wave_id();
    double acc[kRouterTB];
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) acc[t] = 0.0;

    const int nvec = H >> 3;                                   // H % 32 == 0: quarters are whole
    const int q0 = wave * (nvec / kRouterWaves), q1 = q0 + nvec / kRouterWaves;
    for (int v0 = q0 + lane; v0 < q1 + lane; v0 += kWave * kRouterUnroll) {
        u32x4 wv[kRouterUnroll];
#pragma unroll
        for (int u = 0; u < kRouterUnroll; ++u)
            wv[u] = __builtin_nontemporal_load((const u32x4 *)(w) + min(v0 + u * kWave, q1 - 1));
#pragma unroll
        for (int t = 0; t < kRouterTB; ++t) {
            if (t >= nt) break;                      // uniform across the wave
            const u32x4 *xr = (const u32x4 *)(x + (size_t)(t0 + t) * H);
            u32x4 xv[kRouterUnroll];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) xv[u] = xr[min(v0 + u * kWave, q1 - 1)];
            double s = acc[t];
#pragma unroll
            for (int u = 0; u < kRouterUnroll; ++u) {
                if (v0 + u * kWave < q1) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 fw = bf16x2_to_f32x2(wv[u][q]);
                        const f32x2 fx = bf16x2_to_f32x2(xv[u][q]);
                        s = fma((double)fw.x, (double)fx.x, s);
                        s = fma((double)fw.y, (double)fx.y, s);
                    }
                }
            }
            acc[t] = s;
        }
    }
#pragma unroll
    for (int t = 0; t < kRouterTB; ++t) {
        const double s = group_sum_f64(acc[t], kWave);
        if (lane == 0) part[wave][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        double s = 0.0;
#pragma unroll
        for (int w4 = 0; w4 < kRouterWaves; ++w4) s += part[w4][threadIdx.x];
        logits[(size_t)(t0 + threadIdx.x) * rows + row] = (float)s;
    }
}

// Many tokens: a tiled float64 product on the matrix cores.  A workgroup owns 128 tokens x
// 64 rows and one of kRouterKS slices of H; bf16 tiles are converted once to float64 into
// LDS (k-major).  Wave w multiplies tokens 32w .. 32w+31 by the 64 rows with
// v_mfma_f64_16x16x4_f64 (lane l supplies A[l%16][l/16] and B[l/16][l%16]; it receives
// C[l/16 + 4i][l%16]); the products of two bf16 values are exact in float64 and the sums
// are float64.  The next stage's values are loaded while the current one is multiplied.
// The slices' partial sums go to the workspace and router_reduce_kernel adds them in a
// fixed order and rounds once to float32 -- the same logits as the one-wave form, up to
// float64 rounding.
constexpr int kRouterKS = 16;   // K slices
constexpr int kRtTok = 128;     // tokens per tile
constexpr int kRtRow = 64;      // rows per tile
constexpr int kRtKC = 32;       // bf16 values per stage
constexpr int kRtThin = 16;     // row tiles with at most this many rows use plain dot products

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ wr,
                                                              const uint16_t *__restrict__ wsg, int T, int H,
                                                              int E, int rows, double *__restrict__ partial) {
    __shared__ __align__(16) double xs[kRtKC][kRtTok];
    __shared__ __align__(16) double wsm[kRtKC][kRtRow];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * kRtTok, r0 = blockIdx.x * kRtRow;
    const int ks = blockIdx.z;
    const int hs = H / kRouterKS;                      // H % (32 * kRouterKS) is checked on the host
    const int h0 = ks * hs, h1 = h0 + hs;
    auto wrow_of = [&](int r) { return r < E ? wr + (size_t)r * H : wsg; };

    // A tile with few rows (the shared-gate row after a whole number of row tiles, or a
    // small E): each (token, row) pair of the tile is one thread's plain dot product over the
    // slice, in the same order as the tiled form.
    if (rows - r0 <= kRtThin) {
        const int nr = rows - r0;
        for (int i = tid; i < kRtTok * nr; i += 256) {
            const int t = t0 + i / nr, r = r0 + i % nr;
            if (t >= T) continue;
            const uint16_t *xr = x + (size_t)t * H, *wrr = wrow_of(r);
            double s = 0.0;
            for (int h = h0; h < h1; h += 8) {
                const u32x4 xv = *(const u32x4 *)(xr + h), wv = *(const u32x4 *)(wrr + h);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 fx = bf16x2_to_f32x2(xv[q]), fw = bf16x2_to_f32x2(wv[q]);
                    s = fma((double)fx.x, (double)fw.x, s);
                    s = fma((double)fx.y, (double)fw.y, s);
                }
            }
            partial[((size_t)ks * T + t) * rows + r] = s;
        }
        return;
    }

    const int lane = lane_id(), wave = wave_id();
    const int lr = lane & 15, lk = lane >> 4;          // MFMA operand row/column, K index
    // staging (kRtKC = 32 values a stage): x thread -> (token tid/2, 16 values at (tid&1)*16);
    // w thread -> (row tid/4, 8 values at (tid&3)*8)
    const int lt = tid >> 1, lh = (tid & 1) * 16;
    const int lw = tid >> 2, lq = (tid & 3) * 8;
    const int tt = min(t0 + lt, T - 1), rr = min(r0 + lw, rows - 1);
    const bool tok_ok = t0 + lt < T, row_ok = r0 + lw < rows;
    const uint16_t *xrow = x + (size_t)tt * H;
    const uint16_t *wrow = wrow_of(rr);
    f64x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    u32x4 xv0 = *(const u32x4 *)(xrow + h0 + lh), xv1 = *(const u32x4 *)(xrow + h0 + lh + 8);
    u32x4 wv = __builtin_nontemporal_load((const u32x4 *)(wrow + h0 + lq));
    for (int h = h0; h < h1; h += kRtKC) {
        lds_barrier();                                 // the previous stage is consumed
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x2 f0 = bf16x2_to_f32x2(xv0[q]), f1 = bf16x2_to_f32x2(xv1[q]);
            xs[lh + 2 * q][lt] = tok_ok ? (double)f0.x : 0.0;
            xs[lh + 2 * q + 1][lt] = tok_ok ? (double)f0.y : 0.0;
            xs[lh + 8 + 2 * q][lt] = tok_ok ? (double)f1.x : 0.0;
            xs[lh + 8 + 2 * q + 1][lt] = tok_ok ? (double)f1.y : 0.0;
            const f32x2 fw = bf16x2_to_f32x2(wv[q]);
            wsm[lq + 2 * q][lw] = row_ok ? (double)fw.x : 0.0;
            wsm[lq + 2 * q + 1][lw] = row_ok ? (double)fw.y : 0.0;
        }
        const int hn = min(h + kRtKC, h1 - kRtKC);     // (the last stage reloads itself, unused)
        xv0 = *(const u32x4 *)(xrow + hn + lh);
        xv1 = *(const u32x4 *)(xrow + hn + lh + 8);
        wv = __builtin_nontemporal_load((const u32x4 *)(wrow + hn + lq));
        lds_barrier();                                 // (the next stage's loads stay in flight)
#pragma unroll
        for (int k0 = 0; k0 < kRtKC; k0 += 4) {
            double a[2], b[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = xs[k0 + lk][32 * wave + 16 * i + lr];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = wsm[k0 + lk][16 * j + lr];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = t0 + 32 * wave + 16 * i + lk + 4 * v;
            if (t >= T) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 16 * j + lr;
                if (r < rows) partial[((size_t)ks * T + t) * rows + r] = acc[i][j][v];
            }
        }
}

__global__ __launch_bounds__(256) void router_reduce_kernel(const double *__restrict__ partial, int n,
                                                            float *__restrict__ logits) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double s = 0.0;
#pragma unroll
    for (int ks = 0; ks < kRouterKS; ++ks) s += partial[(size_t)ks * n + i];
    logits[i] = (float)s;
}

bool router_tiled(const moe_route_desc *d) { return d->T >= 32 && d->H % (32 * kRouterKS) == 0; }

MOE_DEV double sigmoid_f64(double v) { return 1.0 / (1.0 + exp(-v)); }

MOE_DEV double readlane_f64(double v, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Selection order: larger key first, equal keys (-0 == +0) -> lower expert index.  A key
// is mapped to an unsigned 64-bit integer with the same order (NaN -> 0, below every
// number), so the wave-wide maximum runs on 32-bit integer halves.
MOE_DEV uint64_t order_key(double k) {
    if (k != k) return 0;
    const uint64_t b = (uint64_t)__double_as_longlong(k + 0.0);          // -0 -> +0
    return b ^ ((b >> 63) ? ~0ull : 0x8000000000000000ull);
}

// Maximum of v over the wave, in every lane: a DPP butterfly inside each 16-lane row
// (quad xor 1, quad xor 2, half-row mirror, row mirror), then the four rows via readlane.
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Lane of the wave-wide best (key, index) among the lanes' current heads: the largest high
// key half, then (only on a tie) the largest low half, then the lowest index.
MOE_DEV int wave_best_lane(uint64_t hk, int hi) {
    const uint32_t kh = (uint32_t)(hk >> 32), kl = (uint32_t)hk;
    const uint32_t mh = wave_max_u32(kh);
    uint64_t cand = __ballot(kh == mh);
    if (__popcll(cand) > 1) {
        const bool c1 = kh == mh;
        const uint32_t ml = wave_max_u32(c1 ? kl : 0u);
        cand = __ballot(c1 && kl == ml);
        if (__popcll(cand) > 1) {
            const bool c2 = c1 && kl == ml;
            const uint32_t mi = ~wave_max_u32(c2 ? ~(uint32_t)hi : 0u);   // lowest index
            cand = __ballot(c2 && (uint32_t)hi == mi);
        }
    }
    return __ffsll((long long)cand) - 1;
}

constexpr int kSortNK = 8;                 // most keys per lane that are sorted (more: per-round rescans)

// In-register bitonic sort of a lane's N (power of two) entries into descending order of
// (key, then lower index first); base values move with their keys.
template <int N>
MOE_DEV void sort_desc(uint64_t (&key)[N], int (&idx)[N], double (&base)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int p = i ^ stride;
                if (p <= i) continue;
                // entries i < p: descending run when (i & size) == 0, ascending otherwise
                const bool first_better = key[i] > key[p] || (key[i] == key[p] && idx[i] < idx[p]);
                const bool swap = ((i & size) == 0) ? !first_better : first_better;
                const uint64_t ka = key[i], kb = key[p];
                const int ia = idx[i], ib = idx[p];
                const double ba = base[i], bb = base[p];
                key[i] = swap ? kb : ka;
                key[p] = swap ? ka : kb;
                idx[i] = swap ? ib : ia;
                idx[p] = swap ? ia : ib;
                base[i] = swap ? bb : ba;
                base[p] = swap ? ba : bb;
            }
        }
    }
}

// One wave per token.  Lane l holds the selection keys of experts l, l+64, ... in
// registers; each of the k rounds takes the wave-wide best of the lanes' best untaken keys
// (see the selection below).  NaN keys are never selected (ids -1 are emitted if fewer
// than k keys compare).
// PERM: one workgroup holds every token (T <= 4, T*k <= 64) and also writes the token ->
// expert permutation of the selected ids, as moe_permute would.
template <int NK, bool PERM>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int rows,
                                                   int T, int E, int k, int score, int renorm,
                                                   float scaling, const float *__restrict__ lbias,
                                                   const float *__restrict__ sbias, int has_sg,
                                                   int32_t *__restrict__ ids, float *__restrict__ w,
                                                   float *__restrict__ sg, int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ sorted, int32_t *__restrict__ p2r,
                                                   int n_group, int topk_group) {
    __shared__ int sid[PERM ? 64 : 1];
    extern __shared__ double s_gkey[];      // [4 waves][E] selection keys, group-limited form only
    const int t = blockIdx.x * 4 + wave_id();
    if (!PERM && t >= T) return;
    const int lane = lane_id();
    if (t < T) {
    const float *lt = logits + (size_t)t * rows;

    // All loads are issued before any is used (an absent bias array is read from the logits
    // and the value dropped), so the keys cost one memory round trip.  base[i] is what a
    // selected expert's weight is computed from -- its logit (softmax) or sigmoid (sigmoid)
    // -- so nothing is read again after the selection.
    const float *lbp = lbias ? lbias : lt, *sbp = sbias ? sbias : lt;
    float lv[NK], lbv[NK], sbv[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        lv[i] = lt[e];
        lbv[i] = lbp[e];
        sbv[i] = sbp[e];
    }
    const float sg_logit = lt[has_sg ? E : 0];
#pragma unroll
    for (int i = 0; i < NK; ++i) asm volatile("" : "+v"(lv[i]), "+v"(lbv[i]), "+v"(sbv[i]));   // loads stay here
    uint64_t key[NK];
    double base[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        double l = (double)lv[i] + (lbias ? (double)lbv[i] : 0.0);
        double kv = l;
        if (score == MOE_SCORE_SIGMOID) {
            l = sigmoid_f64(l);
            kv = l + (sbias ? (double)sbv[i] : 0.0);
        }
        base[i] = l;
        key[i] = lane + 64 * i < E ? order_key(kv) : 0;
        if (n_group > 1 && lane + 64 * i < E) s_gkey[wave_id() * E + lane + 64 * i] = kv;
    }
    if (n_group > 1) {
        // group-limited selection: lane g < n_group scores group g from the keys in LDS (a
        // wave's LDS accesses complete in order), the topk_group best groups are taken by
        // wave arg-max rounds, and keys outside them can no longer be selected
        const int gs = E / n_group;
        const double *kw = s_gkey + wave_id() * E;
        double b1 = -INFINITY, b2 = -INFINITY;
        if (lane < n_group) {
            for (int q = 0; q < gs; ++q) {
                double v = kw[lane * gs + q];
                if (v != v) v = -INFINITY;
                if (v > b1) {
                    b2 = b1;
                    b1 = v;
                } else if (v > b2) {
                    b2 = v;
                }
            }
        }
        uint64_t gk = lane < n_group ? order_key(score == MOE_SCORE_SIGMOID ? b1 + b2 : b1) : 0;
        uint64_t keep = 0;
        for (int r = 0; r < topk_group; ++r) {
            const int L = wave_best_lane(gk, lane);
            keep |= 1ull << L;
            if (lane == L) gk = 0;
        }
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((keep >> (e / gs)) & 1ull)) key[i] = 0;
        }
    }
    // Up to kSortNK keys per lane: the lane's keys are sorted once, best first (larger key,
    // then lower expert); each round takes the wave-wide best of the lanes' first entries
    // and the winner shifts its list.  More keys per lane: each lane tracks its best
    // untaken key (its head) and only the round's winner rescans -- the sorting network
    // grows as n log^2 n while the rescans grow as k n.  Both select the same experts in
    // the same order.  Key 0 (NaN, masked or past E) is never selected.
    double braw[NK];             // unsorted, for the full softmax denominator
#pragma unroll
    for (int i = 0; i < NK; ++i) braw[i] = base[i];
    int my_e = -1;
    double l = 0.0;              // lane j < k: base value of the j-th selected expert
    if constexpr (NK <= kSortNK) {
        int idx[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) idx[i] = lane + 64 * i;
        sort_desc<NK>(key, idx, base);
        for (int j = 0; j < k; ++j) {
            const int L = wave_best_lane(key[0], key[0] ? idx[0] : INT_MAX);
            const int wi = key[0] ? idx[0] : INT_MAX;
            const int win = __builtin_amdgcn_readlane(wi, L);
            const double wl = readlane_f64(base[0], L);
            if (lane == j && win != INT_MAX) {
                my_e = win;
                l = wl;
            }
            if (lane == L) {     // the winner drops its first entry
#pragma unroll
                for (int i = 0; i + 1 < NK; ++i) {
                    key[i] = key[i + 1];
                    idx[i] = idx[i + 1];
                    base[i] = base[i + 1];
                }
                key[NK - 1] = 0;
            }
        }
    } else {
        uint32_t taken = 0;
        uint64_t hk;
        int hi;
        double hv;
        auto head = [&]() {      // best untaken key of this lane (equal keys: lower i = lower expert)
            hk = 0;
            hi = INT_MAX;
            hv = 0.0;
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                if (!((taken >> i) & 1u) && key[i] > hk) {
                    hk = key[i];
                    hi = lane + 64 * i;
                    hv = base[i];
                }
            }
        };
        head();
        for (int j = 0; j < k; ++j) {
            const int L = wave_best_lane(hk, hi);
            const int win = __builtin_amdgcn_readlane(hi, L);
            const double wl = readlane_f64(hv, L);
            if (lane == j && win != INT_MAX) {
                my_e = win;
                l = wl;
            }
            if (lane == L && win != INT_MAX) {   // the winner drops its key
                taken |= 1u << (win >> 6);
                head();
            }
        }
    }

    const bool mine = lane < k && my_e >= 0;
    double wv;
    if (score == MOE_SCORE_SOFTMAX) {
        const double lmax = __shfl(l, 0, kWave);   // first selected = largest logit
        double p = mine ? exp(l - lmax) : 0.0;
        double denom;
        if (renorm) {
            denom = group_sum_f64(p, kWave);
        } else {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < NK; ++i)
                if (lane + 64 * i < E) s += exp(braw[i] - lmax);
            denom = group_sum_f64(s, kWave);
        }
        wv = p / denom;
    } else {
        const double sv = mine ? l : 0.0;
        wv = renorm ? sv / group_sum_f64(sv, kWave) : sv;
    }
    wv *= (double)scaling;
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = mine ? (float)wv : NAN;
        if constexpr (PERM) sid[t * k + lane] = my_e;        // -1 when fewer than k keys compare
    }
    if (has_sg && lane == 0) sg[t] = (float)sigmoid_f64((double)sg_logit);
    }
    if constexpr (PERM) {
        lds_barrier();           // sid is in LDS; the id and weight stores need not land first
        small_permutation(sid, T * k, E, offsets, sorted, p2r, threadIdx.x, blockDim.x);
    }
}

moe_status validate_route(const moe_route_desc *d) {
    MOE_REQUIRE(d != nullptr, "moe_route: desc is NULL");
    MOE_REQUIRE(d->T >= 0, "moe_route: T = %d < 0", d->T);
    MOE_REQUIRE(d->H > 0 && d->H % 32 == 0, "moe_route: H = %d must be a positive multiple of 32", d->H);
    MOE_REQUIRE(d->E >= 1 && d->E <= MOE_MAX_EXPERTS, "moe_route: E = %d outside [1, %d]", d->E,
                MOE_MAX_EXPERTS);
    MOE_REQUIRE(d->k >= 1 && d->k <= MOE_MAX_TOPK && d->k <= d->E,
                "moe_route: k = %d outside [1, min(E, %d)]", d->k, MOE_MAX_TOPK);
    MOE_REQUIRE(d->score == MOE_SCORE_SOFTMAX || d->score == MOE_SCORE_SIGMOID,
                "moe_route: unknown score %d", d->score);
    MOE_REQUIRE((int64_t)d->T * (d->E + 1) < INT32_MAX && (int64_t)d->T * d->H < INT32_MAX,
                "moe_route: sizes overflow int32");
    if (d->n_group > 1) {
        const int ng = d->n_group, gs = d->E / ng;
        MOE_REQUIRE(ng <= 64 && d->E % ng == 0, "moe_route: n_group = %d must divide E = %d and be <= 64", ng, d->E);
        MOE_REQUIRE(d->score != MOE_SCORE_SIGMOID || gs >= 2,
                    "moe_route: sigmoid group scores need at least 2 experts per group (E / n_group = %d)", gs);
        MOE_REQUIRE(d->topk_group >= 1 && d->topk_group <= ng && (int64_t)d->topk_group * gs >= d->k,
                    "moe_route: topk_group = %d must be in [1, n_group] and keep at least k experts", d->topk_group);
    } else {
        MOE_REQUIRE(d->n_group >= 0, "moe_route: n_group = %d < 0", d->n_group);
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {

template <bool PERM>
moe_status launch_topk_t(const moe_route_desc *d, const float *logits, int rows, const float *lb, const float *sb,
                         bool has_sg, int32_t *ids, float *w, float *sg, int32_t *offs, int32_t *sorted,
                         int32_t *p2r, hipStream_t s) {
    auto topk = d->E <= 256 ? topk_kernel<4, PERM> : d->E <= 512 ? topk_kernel<8, PERM>
              : d->E <= 1024 ? topk_kernel<16, PERM> : topk_kernel<32, PERM>;
    const int tb = (d->T < 4 && !PERM) ? 64 * d->T : 256;   // the permutation uses every thread
    const int ng = d->n_group > 1 ? d->n_group : 1;
    const size_t lds = ng > 1 ? (size_t)(tb / 64) * d->E * sizeof(double) : 0;
    hipLaunchKernelGGL(topk, dim3((d->T + 3) / 4), dim3(tb), lds, s, logits, rows, d->T, d->E, d->k, d->score,
                       d->renormalize, d->routed_scaling, lb, sb, has_sg ? 1 : 0, ids, w, sg, offs, sorted, p2r, ng,
                       ng > 1 ? d->topk_group : 1);
    return launch_check(PERM ? "moe_route_permute: topk_kernel" : "moe_route: topk_kernel");
}

moe_status launch_topk(const moe_route_desc *d, const float *logits, int rows, const float *lb, const float *sb,
                       bool has_sg, int32_t *ids, float *w, float *sg, int32_t *offs, int32_t *sorted, int32_t *p2r,
                       hipStream_t s) {
    if (offs) return launch_topk_t<true>(d, logits, rows, lb, sb, has_sg, ids, w, sg, offs, sorted, p2r, s);
    return launch_topk_t<false>(d, logits, rows, lb, sb, has_sg, ids, w, sg, nullptr, nullptr, nullptr, s);
}

}  // namespace

extern "C" size_t moe_route_workspace(const moe_route_desc *d) {
    if (!d || d->T <= 0 || d->E <= 0) return 0;
    size_t b = align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256);
    if (d->H % 32 == 0 && router_tiled(d)) b += (size_t)kRouterKS * d->T * (d->E + 1) * sizeof(double);
    return b;
}

namespace {

// Checks the routing arguments and enqueues the logits (router_logits_kernel, or the tiled
// product and its reduction) into the workspace.
moe_status route_logits(const moe_route_desc *d, const void *x, const void *w_router, const float *logit_bias,
                        const float *select_bias, const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                        float *shared_gate, void *ws, size_t ws_bytes, hipStream_t s) {
    MOE_REQUIRE(x && w_router && topk_ids && topk_w, "moe_route: NULL x, w_router, topk_ids or topk_w");
    MOE_REQUIRE(!(select_bias && d->score != MOE_SCORE_SIGMOID),
                "moe_route: select_bias is only defined for MOE_SCORE_SIGMOID");
    MOE_REQUIRE((w_shared_gate == nullptr) == (shared_gate == nullptr),
                "moe_route: w_shared_gate and shared_gate must both be given or both NULL");
    const size_t need = moe_route_workspace(d);
    if (!ws || ws_bytes < need) {
        set_error("moe_route: workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
        return MOE_ERR_WORKSPACE;
    }
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    float *logits = (float *)ws;
    if (router_tiled(d)) {
        double *partial = (double *)((unsigned char *)ws + align_up((size_t)d->T * (d->E + 1) * sizeof(float), 256));
        dim3 gt((rows + kRtRow - 1) / kRtRow, (d->T + kRtTok - 1) / kRtTok, kRouterKS);
        hipLaunchKernelGGL(router_tiled_kernel, gt, dim3(256), 0, s, (const uint16_t *)x, (const uint16_t *)w_router,
                           (const uint16_t *)w_shared_gate, d->T, d->H, d->E, rows, partial);
        MOE_TRY(launch_check("moe_route: router_tiled_kernel"));
        const int n = d->T * rows;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, partial, n, logits);
        MOE_TRY(launch_check("moe_route: router_reduce_kernel"));
    } else {
        dim3 g1(rows, (d->T + kRouterTB - 1) / kRouterTB);
        hipLaunchKernelGGL(router_logits_kernel, g1, dim3(64 * kRouterWaves), 0, s, (const uint16_t *)x,
                           (const uint16_t *)w_router, (const uint16_t *)w_shared_gate, d->T, d->H, d->E,
                           rows, logits);
        MOE_TRY(launch_check("moe_route: router_logits_kernel"));
    }
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_route(const moe_route_desc *d, const void *x, const void *w_router,
                                const float *logit_bias, const float *select_bias,
                                const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                float *shared_gate, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    if (d->T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(route_logits(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate, ws,
                         ws_bytes, s));
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    return launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                       topk_w, shared_gate, nullptr, nullptr, nullptr, s);
}

extern "C" moe_status moe_route_permute(const moe_route_desc *d, const void *x, const void *w_router,
                                        const float *logit_bias, const float *select_bias,
                                        const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                        float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                        int32_t *pair_to_row, void *ws, size_t ws_bytes, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    MOE_REQUIRE(expert_offsets != nullptr, "moe_route_permute: NULL expert_offsets");
    MOE_REQUIRE((int64_t)d->T * d->k < INT32_MAX, "moe_route_permute: T*k overflows int32");
    if (d->T > 0) MOE_REQUIRE(sorted_pairs && pair_to_row, "moe_route_permute: NULL sorted_pairs or pair_to_row");
    hipStream_t s = (hipStream_t)stream;
    if (d->T == 0) return moe_permute(0, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0,
                                      stream);
    MOE_TRY(route_logits(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate, ws,
                         ws_bytes, s));
    const int rows = d->E + (w_shared_gate ? 1 : 0);
    if (d->T <= 4 && d->T * d->k <= 64)      // one workgroup holds every token: fused permutation
        return launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                           topk_w, shared_gate, expert_offsets, sorted_pairs, pair_to_row, s);
    MOE_TRY(launch_topk(d, (const float *)ws, rows, logit_bias, select_bias, w_shared_gate != nullptr, topk_ids,
                        topk_w, shared_gate, nullptr, nullptr, nullptr, s));
    return moe_permute(d->T, d->k, d->E, topk_ids, expert_offsets, sorted_pairs, pair_to_row, nullptr, 0, stream);
}

// ------------------------------------------------------------------ no-allocation entry point
// moe_route_permute_noalloc keeps the routing scratch (float32 logits, and for the tiled
// router its float64 split-K partials) in this file-scope device array instead of a
// caller-provided workspace.  Each GPU holds its own copy, at its own address, until the
// process ends; host code uses that address (from hipGetSymbolAddress, once per device),
// never the array's name.  Every call on a GPU shares the array: the kernels overwrite all
// of it that they read, so nothing needs clearing, and calls that overlap on one GPU race.
constexpr size_t kRouteScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kScratchMaxDevices] = {};

// This device's address of `scratch`, looked up on its first use with the device current.
moe_status route_scratch(void **out) {
    int dev = -1;
    MOE_TRY(hip_check(hipGetDevice(&dev), "moe_route_permute_noalloc: hipGetDevice"));
    if (dev < 0 || dev >= kScratchMaxDevices) {
        set_error("moe_route_permute_noalloc: device %d outside [0, %d)", dev, kScratchMaxDevices);
        return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        MOE_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "moe_route_permute_noalloc: hipGetSymbolAddress"));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_route_permute_noalloc(const moe_route_desc *d, const void *x, const void *w_router,
                                                const float *logit_bias, const float *select_bias,
                                                const void *w_shared_gate, int32_t *topk_ids, float *topk_w,
                                                float *shared_gate, int32_t *expert_offsets, int32_t *sorted_pairs,
                                                int32_t *pair_to_row, moe_stream stream) {
    clear_error();
    MOE_TRY(validate_route(d));
    const size_t need = moe_route_workspace(d);
    if (need > kRouteScratchBytes) {
        set_error("moe_route_permute_noalloc: T = %d, E = %d need %zu bytes of scratch, more than the %zu it holds",
                  d->T, d->E, need, kRouteScratchBytes);
        return MOE_ERR_UNSUPPORTED;
    }
    void *ws = nullptr;
    if (d->T > 0) MOE_TRY(route_scratch(&ws));
    return moe_route_permute(d, x, w_router, logit_bias, select_bias, w_shared_gate, topk_ids, topk_w, shared_gate,
                             expert_offsets, sorted_pairs, pair_to_row, ws, kRouteScratchBytes, stream);
}

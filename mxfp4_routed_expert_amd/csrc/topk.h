// Top-k selection of one token's routing in one wave, shared by the route kernel and the
// decode gate/up kernel that routes in its prologue.
//
// Routing schemes of the pages: "softmax top-10 of 512 + gated shared expert"
// (Qwen3.8-Max) and "noaux_tc sigmoid" (GLM-5.2) -- rabbit README, architecture table,
// "MoE routing" row.  Scoring, top-k and the weights run in float64; only the final
// weights are rounded to float32.
#pragma once

#include <limits.h>
#include <math.h>

#include "common.h"

namespace moe {

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
constexpr int kSortPackedNK = 16;          // ... for packed words, which sort with one compare per exchange

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

// Softmax scores without a logit bias select on float32 logits, whose order a 32-bit key
// carries exactly (NaN -> 0, below every number; -0 == +0).  Packed with the bitwise NOT of
// the expert index in the low half, one 64-bit word orders (larger logit, then lower expert)
// and holds both, so the sort and the k rounds move one value per entry instead of a key, an
// index and a float64 base value.  A word with a zero high half is never selected.
MOE_DEV uint32_t order_key32(float v) {
    if (v != v) return 0u;
    const uint32_t b = __float_as_uint(v + 0.0f);                         // -0 -> +0
    return b ^ ((b >> 31) ? 0xffffffffu : 0x80000000u);
}
MOE_DEV float key32_value(uint32_t k) {
    return __uint_as_float((k >> 31) ? (k ^ 0x80000000u) : ~k);
}

template <int N>
MOE_DEV void sort_desc_packed(uint64_t (&key)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
        for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int p = i ^ stride;
                if (p <= i) continue;
                const bool swap = ((i & size) == 0) ? key[i] < key[p] : key[i] > key[p];
                const uint64_t ka = key[i], kb = key[p];
                key[i] = swap ? kb : ka;
                key[p] = swap ? ka : kb;
            }
        }
    }
}

// One token's selection in one wave.  Lane l holds the selection keys of experts l, l+64,
// ... (NK per lane, E <= 64 * NK) in registers; each of the k rounds takes the wave-wide best
// of the lanes' best untaken keys.  NaN keys are never selected.  lt: the token's logits
// (E, then the shared-gate logit when has_sg); gkey: E doubles of LDS for this wave
// (group-limited selection only).  Returns, in lane j < k, the j-th selected expert (-1 when
// fewer than k keys compare) and its routing weight (NaN then); in every lane, the shared
// gate sigmoid(logit) when has_sg.
struct TopkLane {
    int e;
    float w;
    float sg;
};

template <int NK>
MOE_DEV TopkLane topk_select(const float *lt, int E, int k, int score, int renorm, float scaling,
                             const float *lbias, const float *sbias, int has_sg, double *gkey, int n_group,
                             int topk_group) {
    const int lane = lane_id();
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
    const bool packed = NK <= kSortPackedNK && score == MOE_SCORE_SOFTMAX && !lbias && n_group <= 1;
    uint64_t key[NK];
    double base[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        if (packed) {                // (the packed words below carry the keys; base: the full softmax sum)
            base[i] = (double)lv[i] + 0.0;
            key[i] = 0;
            continue;
        }
        double l = (double)lv[i] + (lbias ? (double)lbv[i] : 0.0);
        double kv = l;
        if (score == MOE_SCORE_SIGMOID) {
            l = sigmoid_f64(l);
            kv = l + (sbias ? (double)sbv[i] : 0.0);
        }
        base[i] = l;
        key[i] = lane + 64 * i < E ? order_key(kv) : 0;
        if (n_group > 1 && lane + 64 * i < E) gkey[lane + 64 * i] = kv;
    }
    if (n_group > 1) {
        // group-limited selection: lane g < n_group scores group g from the keys in LDS (a
        // wave's LDS accesses complete in order), the topk_group best groups are taken by
        // wave arg-max rounds, and keys outside them can no longer be selected
        const int gs = E / n_group;
        const double *kw = gkey;
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
    // Up to kSortNK keys per lane (kSortPackedNK packed words): the lane's keys are sorted
    // once, best first (larger key,
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
    if (packed) {
        // keys from the loaded float logits (the same order as order_key of their float64 values)
        uint64_t pk[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int e = lane + 64 * i;
            const uint32_t k32 = e < E ? order_key32(lv[i]) : 0u;
            pk[i] = k32 ? ((uint64_t)k32 << 32) | (uint32_t)~e : 0ull;
        }
        sort_desc_packed<NK>(pk);
        for (int j = 0; j < k; ++j) {
            // (low halves are distinct, so the wave-wide maximum is one lane's word)
            const int L = wave_best_lane(pk[0], 0);
            const uint32_t wh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pk[0] >> 32), L);
            const uint32_t wl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pk[0], L);
            if (lane == j && wh != 0u) {
                my_e = (int)~wl;
                l = (double)key32_value(wh);
            }
            if (lane == L) {     // the winner drops its first entry
#pragma unroll
                for (int i = 0; i + 1 < NK; ++i) pk[i] = pk[i + 1];
                pk[NK - 1] = 0ull;
            }
        }
    } else if constexpr (NK <= kSortNK) {
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
    TopkLane r;
    r.e = lane < k ? my_e : -1;
    r.w = mine ? (float)wv : NAN;
    r.sg = has_sg ? (float)sigmoid_f64((double)sg_logit) : 0.0f;
    return r;
}

}  // namespace moe

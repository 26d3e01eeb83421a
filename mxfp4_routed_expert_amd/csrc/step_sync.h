// Hand-offs between the phases of the single-launch decode step (decode_step_kernel):
// router logits -> top-k and gate/up -> down and combine.  Every workgroup of the launch is
// resident at once (one per compute unit), so a phase can wait for all of them.
//
// The caller owns a small device buffer (moe_decode_step_sync_bytes(), zero-filled once):
// word 0 counts the launches that used it, word 1 is an error word, words kSyncFlag0 + b
// are workgroup b's arrival flags and from word kSyncLogit0 on lie the launch's tagged
// logits.  A launch reads the count c at its start.
//
// Logits -> top-k: every logit is also stored as one 64-bit word (c + 1) << 32 | its float
// bits, by a device-scope atomic store; a routing wave reads its token's words with
// device-scope atomic loads until every tag is c + 1.  The data carries its own readiness,
// so this hand-off costs no fence and no second read.
//
// h rows -> down: h is written with device-scope atomic stores (step_put) and read with
// device-scope atomic loads (step_get4), which the compute dies' separate L2 caches keep
// coherent without a cache write-back or invalidation.  Workgroup b announces that its h
// rows are stored by storing c + 1 into its flag once every wave has waited for its h
// stores to complete; the down phase waits until every flag has reached c + 1.
//
// Counts, tags and flags only grow from one launch to the next, so nothing is ever reset,
// and a captured graph replays correctly (the count lives in device memory, not in the
// kernel arguments).  Workgroup 0 stores c + 1 into word 0 once every workgroup has arrived
// at the h hand-off, by which time every workgroup has read c.  Waits are bounded: past the
// bound the wave sets the error word and goes on, so a fault elsewhere cannot turn into a
// hang; the results of such a launch are undefined.
#pragma once

#include "common.h"

namespace moe {

constexpr int kSyncFlag0 = 64;                 // first flag word (the counters have a line of their own)
constexpr int kSyncMaxWG = 1024;               // flags in the buffer
constexpr int kSyncLogit0 = kSyncFlag0 + kSyncMaxWG;   // tagged logits, 64-bit words
constexpr int kSyncMaxT = 4;                   // tokens of a single launch
constexpr int kSyncRowStride = 520;            // tagged words per token (>= E + 1, E <= 512)
constexpr int kSyncWords = kSyncLogit0 + 2 * kSyncMaxT * kSyncRowStride;
constexpr int kSyncSpin = 1 << 15;             // polls before a wait gives up (tens of ms)

struct StepRouting {                           // a workgroup's own routing, kept in LDS for the down phase
    float lt[kSyncMaxT][kSyncRowStride];       // the logits the routing waves collected
    int ids[64];                               // expert of pair t*k + j (-1: dropped)
    int p2r[64];                               // its row in the sorted order
    float tw[64];                              // its weight
    float sg[4];                               // shared gate of token t
};

struct StepCtx {
    uint32_t *sync;                            // the caller's buffer
    uint32_t tag;                              // c + 1: the logits' tag and the flag value of the h hand-off
    int nwg;
    StepRouting *lds;
};

MOE_DEV uint32_t step_launch_count(const uint32_t *sync) {
    return __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread: store logit (token t, row r) as its tagged word.
MOE_DEV void step_put_logit(uint32_t *sync, uint32_t tag, int t, int r, float v) {
    uint64_t *w = (uint64_t *)(sync + kSyncLogit0) + (size_t)t * kSyncRowStride + r;
    __hip_atomic_store(w, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One whole wave: collect the `rows` tagged logits of token t into dst (LDS), reading until
// every word carries `tag`.
MOE_DEV void step_get_logits(uint32_t *sync, uint32_t tag, int t, int rows, float *dst) {
    constexpr int NV = (kSyncRowStride + kWave - 1) / kWave;
    const int lane = lane_id();
    const uint64_t *src = (const uint64_t *)(sync + kSyncLogit0) + (size_t)t * kSyncRowStride;
    uint64_t v[NV];
    for (int spin = 0;; ++spin) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i] = __hip_atomic_load(src + min(lane + kWave * i, rows - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && (uint32_t)(v[i] >> 32) == tag;
        }
        if (__ballot(!ok) == 0ull) break;
        if (spin >= kSyncSpin) {
            if (lane == 0) __hip_atomic_store(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (lane + kWave * i < rows) dst[lane + kWave * i] = __uint_as_float((uint32_t)v[i]);
}

// h values: stored and loaded at device scope.
MOE_DEV void step_put(float *dst, float v) {
    __hip_atomic_store((uint32_t *)dst, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV f32x4 step_get4(const float *src) {                  // 16-byte aligned
    const uint64_t a = __hip_atomic_load((const uint64_t *)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load((const uint64_t *)src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
                 __uint_as_float((uint32_t)(b >> 32))};
}

// One thread of the workgroup, after a barrier that follows every wave's wait for its h
// stores: raise the workgroup's flag.
MOE_DEV void step_flag(uint32_t *sync, uint32_t value) {
    __hip_atomic_store(sync + kSyncFlag0 + blockIdx.x, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One whole wave: wait until the flags of workgroups 0 .. nwg-1 have reached `value`.
MOE_DEV void step_wait(uint32_t *sync, int nwg, uint32_t value) {
    const int lane = lane_id();
    for (int spin = 0;; ++spin) {
        bool ok = true;
        for (int i = lane; i < nwg; i += kWave) {
            const uint32_t f = __hip_atomic_load(sync + kSyncFlag0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && (int32_t)(f - value) >= 0;
        }
        if (__ballot(!ok) == 0ull) break;
        if (spin >= kSyncSpin) {
            if (lane == 0) __hip_atomic_store(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

}  // namespace moe

// Hand-offs between the phases of the single-launch decode step (decode_step_kernel):
// router logits -> top-k and gate/up -> down and combine.  Every workgroup of the launch is
// resident at once (one per compute unit), so a phase can wait for all of them.
//
// The caller owns a small device buffer (moe_decode_step_sync_bytes(), zero-filled once):
// word 0 is the launch count, word 1 an error word, and words kSyncFlag0 + b are workgroup
// b's arrival flags.  A launch reads the count c at its start and workgroup b announces the
// end of phase q (1, 2) by storing 2c + q into its flag; a phase waits until every flag has
// reached that value.  The values only grow from one launch to the next, so no flag is ever
// reset, and a captured graph replays correctly (the count lives in device memory, not in
// the kernel arguments).  Workgroup 0 stores c + 1 once every workgroup has arrived at the
// end of phase 2, by which time every workgroup has read c.
//
// Memory ordering: the writers of a phase's results wait for their stores, the workgroup
// meets at a barrier, and one thread releases at device scope (the write-back of the
// compute die's L2) before storing the flag; a waiting wave reads the flags with
// device-scope loads and then acquires at device scope (the invalidation of the CU's L1 and
// of its die's L2), so what it reads next is what the other workgroups wrote.  Waits are
// bounded: past the bound the wave sets the error word and goes on, so a fault elsewhere
// cannot turn into a hang; the results of such a launch are undefined.
#pragma once

#include "common.h"

namespace moe {

constexpr int kSyncFlag0 = 64;                 // first flag word (the counters have a line of their own)
constexpr int kSyncMaxWG = 1024;               // flags in the buffer
constexpr int kSyncWords = kSyncFlag0 + kSyncMaxWG;
constexpr int kSyncSpin = 1 << 15;             // polls before a wait gives up (tens of ms)

struct StepRouting {                           // a workgroup's own routing, kept in LDS for the down phase
    int ids[64];                               // expert of pair t*k + j (-1: dropped)
    int p2r[64];                               // its row in the sorted order
    float tw[64];                              // its weight
    float sg[4];                               // shared gate of token t
};

struct StepCtx {
    uint32_t *sync;                            // the caller's buffer
    uint32_t target_logits, target_h;          // flag values that end phases 1 and 2
    int nwg;
    StepRouting *lds;
};

MOE_DEV uint32_t step_launch_count(const uint32_t *sync) {
    return __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread of the workgroup, after a barrier that follows every writer's wait for its
// stores: make the workgroup's writes visible at device scope, then raise its flag.
MOE_DEV void step_arrive(uint32_t *sync, uint32_t value) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(sync + kSyncFlag0 + blockIdx.x, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One whole wave: wait until the flags of workgroups 0 .. nwg-1 have reached `value`, then
// acquire at device scope.  Returns after the acquisition has completed (its wait on the
// vector memory counter also waits for the wave's loads in flight).
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
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace moe

// Shared helpers of the HIP library: device-side number decoding, wave reductions,
// host-side error reporting and argument checks.  gfx950 (CDNA4) only: 64-lane
// wavefronts, the scaled FP4/FP8 conversion instructions and the block-scaled MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "moe.h"

#define MOE_DEV __device__ __forceinline__

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ device decoding

MOE_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bf16 bits, rounded to nearest even; NaN stays NaN.
MOE_DEV uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // NaN stays NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// E8M0 scale byte -> float32 2^(b-127).  b = 0 is the float32 subnormal 2^-127;
// b = 255 is NaN (OCP MX v1.0, E8M0).
MOE_DEV float e8m0_to_f32(uint32_t b) {
    uint32_t bits = b == 0 ? 0x00400000u : (b == 255 ? 0x7fc00000u : (b << 23));
    return __uint_as_float(bits);
}

// Four bf16 pairs -> one 8-value operand slice, in order.
MOE_DEV bf16x8 pack8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// The scaled MXFP4 decode of every kernel that multiplies decoded weights (or MX-encoded
// activations) in bf16: eight E2M1 codes of one dword (byte b holds elements 2b, 2b+1,
// low nibble first) times the block scale `sc` (2^(s-127), e8m0_to_f32), by the gfx950
// scaled conversion, which applies the scale inside the instruction.  An E2M1 value times
// a power of two is a bf16 value unless it leaves bf16's range; moe_dequant_bf16 runs this
// same function, so its output is what the kernels multiply.
MOE_DEV bf16x8 fp4x8_scaled_bf16(uint32_t w, float sc) {
    return pack8(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1),
                 __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2), __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
}
// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}): an unrolled
// loop whose index is a constant expression, so per-iteration register arrays indexed by it
// stay in registers.
template <class F, int... Ds>
MOE_DEV void static_for_impl(F &&f, std::integer_sequence<int, Ds...>) {
    (f(std::integral_constant<int, Ds>{}), ...);
}
template <int N, class F>
MOE_DEV void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Loads through the global address space.  A pointer that reaches a load through a struct
// or a select may lose its address space; the compiler then emits flat loads, which count
// against the LDS wait counter too, so every LDS access waits for every load in flight.
#define MOE_GLOBAL __attribute__((address_space(1)))
MOE_DEV u32x4 gload16_nt(const void *p) { return __builtin_nontemporal_load((const MOE_GLOBAL u32x4 *)p); }
MOE_DEV uint32_t gload_u8(const void *p) { return *(const MOE_GLOBAL uint8_t *)p; }
MOE_DEV uint32_t gload_u32(const void *p) { return *(const MOE_GLOBAL uint32_t *)p; }
MOE_DEV int gload_i32(const void *p) { return *(const MOE_GLOBAL int *)p; }

MOE_DEV u32x4 fp4x8_scaled_bf16_bits(uint32_t w, float sc) { return __builtin_bit_cast(u32x4, fp4x8_scaled_bf16(w, sc)); }

// MFMA operand slices of one 32-code MXFP4 unit with its block scale: slice q = values 8q..8q+7.
MOE_DEV void unit_to_bf16x8(const u32x4 w, float sc, bf16x8 (&a)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = fp4x8_scaled_bf16(w[q], sc);
}

// Two E2M1 codes (byte `sel` of `w`: low nibble first) -> two bf16 values, unscaled.
// E2M1 magnitudes (0 .. 6) are exact in bf16.
template <int SEL>
MOE_DEV bf16x2 fp4x2_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
template <int SEL>
MOE_DEV f32x2 fp4x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
// Two E4M3 codes (16-bit half `HI` of `w`, low byte first) -> two values, unscaled.
template <bool HI>
MOE_DEV bf16x2 fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
template <bool HI>
MOE_DEV f32x2 fp8x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
}
// bf16 pair (packed in a dword, low half first) -> two floats.
MOE_DEV f32x2 bf16x2_to_f32x2(uint32_t w) {
    f32x2 r;
    r.x = __uint_as_float(w << 16);
    r.y = __uint_as_float(w & 0xffff0000u);
    return r;
}
MOE_DEV bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

MOE_DEV float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// silu(g) = g / (1 + exp(-g)); finite for every finite g (exp overflow gives -0).
MOE_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------------------ wave reductions
// Butterfly sums over aligned groups of `width` lanes (power of two <= 64); every lane
// of the group ends with the same value, summed in the same order on every run.
MOE_DEV float group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
MOE_DEV double group_sum_f64(double v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

MOE_DEV int lane_id() { return threadIdx.x & (kWave - 1); }

// Workgroup barrier for LDS traffic only: this wave's LDS accesses are complete, then all
// waves meet.  Unlike __syncthreads it does not wait for the wave's global loads in flight.
MOE_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
MOE_DEV int wave_id() { return threadIdx.x >> 6; }

constexpr int kMaxOffsetChunks = MOE_MAX_EXPERTS / 64 + 1;

// Index of the slot-th expert that owns rows (same value in every lane), -1 if none.
// All offsets are loaded in one batch of independent loads, so the lookup costs one
// memory round trip; no LDS and no barrier.
MOE_DEV int wave_nth_nonempty(const int32_t *offsets, int E, int slot, int *row0 = nullptr, int *rows = nullptr) {
    const int lane = lane_id();
    int o[kMaxOffsetChunks];
#pragma unroll
    for (int c = 0; c < kMaxOffsetChunks; ++c) {
        const int i = c * 64 + lane;
        o[c] = i <= E ? offsets[i] : 0;
    }
    int base = 0;
#pragma unroll
    for (int c = 0; c < kMaxOffsetChunks; ++c) {
        if (c * 64 >= E) break;
        const int next = c + 1 < kMaxOffsetChunks ? __shfl(o[c + 1], 0, kWave) : 0;
        int o1 = __shfl_down(o[c], 1, kWave);
        if (lane == 63) o1 = next;
        const int e = c * 64 + lane;
        const bool ne = e < E && o1 > o[c];
        const uint64_t m = __ballot(ne);
        const int cnt = __popcll(m);
        if (slot < base + cnt) {
            const int before = __popcll(m & ((1ull << lane) - 1ull));
            const uint64_t hit = __ballot(ne && before == slot - base);
            const int l = __ffsll((long long)hit) - 1;
            // the expert's first row and row count come from the offsets already loaded
            const int r0 = __builtin_amdgcn_readfirstlane(__shfl(o[c], l, kWave));
            if (row0) *row0 = r0;
            if (rows) *rows = __builtin_amdgcn_readfirstlane(__shfl(o1, l, kWave)) - r0;
            return c * 64 + l;
        }
        base += cnt;
    }
    return -1;
}

// Token -> expert permutation of few pairs (P <= 64) by one workgroup of nthreads threads;
// sid[0..P) in LDS holds the pairs' expert ids, already set to -1 where outside [0, E).
// The stable rank of pair p is the number of valid pairs q with (id_q, q) < (id_p, p);
// expert e's first row is the number of valid ids below e.  Every thread first copies the
// ids to registers (CAP >= P slots, independent LDS reads), so the counting loops run on
// registers.  Needs a barrier between the writes of sid and the call; ends without one.
constexpr int kSmallPermMax = 64;
template <int CAP>
MOE_DEV void small_permutation_t(const int *sid, int P, int E, int32_t *offsets, int32_t *sorted, int32_t *p2r,
                                 int tid, int nthreads) {
    int id[CAP];
#pragma unroll
    for (int q = 0; q < CAP; ++q) id[q] = q < P ? sid[q] : -1;
    int nvalid = 0;
#pragma unroll
    for (int q = 0; q < CAP; ++q) nvalid += id[q] >= 0;
    for (int pp = tid; pp < P; pp += nthreads) {
        int me = -1;
#pragma unroll
        for (int q = 0; q < CAP; ++q) me = q == pp ? id[q] : me;
        if (me < 0) {
            p2r[pp] = -1;
        } else {
            int r = 0;
#pragma unroll
            for (int q = 0; q < CAP; ++q) r += id[q] >= 0 && (id[q] < me || (id[q] == me && q < pp));
            sorted[r] = pp;
            p2r[pp] = r;
        }
    }
    for (int e = tid; e <= E; e += nthreads) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < CAP; ++q) c += id[q] >= 0 && id[q] < e;
        offsets[e] = c;
    }
    for (int r = nvalid + tid; r < P; r += nthreads) sorted[r] = -1;
}
MOE_DEV void small_permutation(const int *sid, int P, int E, int32_t *offsets, int32_t *sorted, int32_t *p2r,
                               int tid, int nthreads) {
    if (P <= 16) small_permutation_t<16>(sid, P, E, offsets, sorted, p2r, tid, nthreads);
    else small_permutation_t<kSmallPermMax>(sid, P, E, offsets, sorted, p2r, tid, nthreads);
}

}  // namespace moe

// ------------------------------------------------------------------ host side
namespace moe {

void set_error(const char *fmt, ...);
void clear_error();
moe_status hip_check(hipError_t e, const char *what);
moe_status launch_check(const char *what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// Compute units of the current device (queried once per device; 256 if the query fails).
int device_cu_count();

}  // namespace moe

#define MOE_REQUIRE(cond, ...)                                       \
    do {                                                             \
        if (!(cond)) {                                               \
            ::moe::set_error(__VA_ARGS__);                           \
            return MOE_ERR_INVALID_ARG;                              \
        }                                                            \
    } while (0)

#define MOE_TRY(expr)                      \
    do {                                   \
        moe_status _st = (expr);           \
        if (_st != MOE_OK) return _st;     \
    } while (0)

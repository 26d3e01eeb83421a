// OCP MX quantisation of activation rows, and weight decoding to float32.
//
// The pages only name the format ("OCP MXFP4", rabbit README architecture table); the
// conversion of a 32-value block follows the OCP Microscaling Formats v1.0 rule:
//   X = floor(log2(max|v|)) - 2 (2 = largest E2M1 exponent), kept in [-127, 127];
//   each v / 2^X goes to the nearest E2M1 value, ties to an even code, saturating at 6.
// Here the rounding is done by counting the E2M1 midpoints a magnitude passes; a
// midpoint whose tie goes to the upper (even) code is tested with >=, the others with >.
#include "gemv.h"

namespace moe {

// E2M1 code (0..7) of a non-negative scaled magnitude a (a = |v| / 2^X < 8).
MOE_DEV uint32_t e2m1_rne_code(float a) {
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
           (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// Quantise one 32-value block held as 32 floats.  Writes 16 code bytes and returns the
// scale byte.
MOE_DEV uint32_t mx_quantize_block(const float *v, uint32_t *codes4) {
    uint32_t amax_bits = 0;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
        bad |= b >= 0x7f800000u;                 // Inf or NaN
        amax_bits = b > amax_bits ? b : amax_bits;
    }
    if (bad) {
#pragma unroll
        for (int d = 0; d < 4; ++d) codes4[d] = 0;
        return 255;
    }
    const int ebits = (int)(amax_bits >> 23);     // biased exponent of max|v|
    int X = ebits == 0 ? -127 : ebits - 127 - 2;  // zero or subnormal max -> the smallest scale
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, X in [-127, 125]
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float x = v[8 * d + q];
            const uint32_t sign = (__float_as_uint(x) >> 31) << 3;
            const uint32_t c = e2m1_rne_code(fabsf(x) * inv) | sign;
            word |= c << (4 * q);
        }
        codes4[d] = word;
    }
    return (uint32_t)(X + 127);
}

namespace {

template <bool F32>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void *__restrict__ x, int rows, int cols,
                                                          uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales) {
    const int nb = cols / 32;
    const long long blk = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= (long long)rows * nb) return;
    float v[32];
    if constexpr (F32) {
        const f32x4 *src = (const f32x4 *)((const float *)x + blk * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 q = src[i];
            v[4 * i] = q[0]; v[4 * i + 1] = q[1]; v[4 * i + 2] = q[2]; v[4 * i + 3] = q[3];
        }
    } else {
        const u32x4 *src = (const u32x4 *)((const uint16_t *)x + blk * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 q = src[i];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x2 f = bf16x2_to_f32x2(q[d]);
                v[8 * i + 2 * d] = f.x;
                v[8 * i + 2 * d + 1] = f.y;
            }
        }
    }
    uint32_t c[4];
    const uint32_t s = mx_quantize_block(v, c);
    ((u32x4 *)codes)[blk] = u32x4{c[0], c[1], c[2], c[3]};
    scales[blk] = (uint8_t)s;
}

// Decode one 16-byte unit per thread with the conversions of the decode GEMV: each code
// unscaled to float32 (E2M1 and E4M3 values are exact), times the block scale in float32.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales, int n, int kdim,
                                                      float *__restrict__ out) {
    const int upr = FMT == 0 ? kdim / 32 : kdim / 16;
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= (long long)n * upr) return;
    const int row = (int)(u / upr), b = (int)(u - (long long)row * upr);
    const u32x4 wv = ((const u32x4 *)codes)[u];
    if constexpr (FMT == 0) {
        const float sc = e8m0_to_f32(((const uint8_t *)scales)[u]);
        float *o = out + (size_t)row * kdim + (size_t)b * 32;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x2 w0 = fp4x2_to_f32x2<0>(wv[d]), w1 = fp4x2_to_f32x2<1>(wv[d]);
            const f32x2 w2 = fp4x2_to_f32x2<2>(wv[d]), w3 = fp4x2_to_f32x2<3>(wv[d]);
            o[8 * d + 0] = w0.x * sc; o[8 * d + 1] = w0.y * sc;
            o[8 * d + 2] = w1.x * sc; o[8 * d + 3] = w1.y * sc;
            o[8 * d + 4] = w2.x * sc; o[8 * d + 5] = w2.y * sc;
            o[8 * d + 6] = w3.x * sc; o[8 * d + 7] = w3.y * sc;
        }
    } else {
        const float sc = ((const float *)scales)[(size_t)(row / 128) * (kdim / 128) + (b * 16) / 128];
        float *o = out + (size_t)row * kdim + (size_t)b * 16;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x2 w0 = fp8x2_to_f32x2<false>(wv[d]), w1 = fp8x2_to_f32x2<true>(wv[d]);
            o[4 * d + 0] = w0.x * sc; o[4 * d + 1] = w0.y * sc;
            o[4 * d + 2] = w1.x * sc; o[4 * d + 3] = w1.y * sc;
        }
    }
}

// MXFP4 unit -> 32 bf16 values with the scaled conversion of the matrix-core kernels
// (fp4x8_scaled_bf16), one 16-byte unit per thread.
__global__ __launch_bounds__(256) void dequant_bf16_kernel(const uint8_t *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales, long long units,
                                                           uint16_t *__restrict__ out) {
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= units) return;
    const u32x4 wv = ((const u32x4 *)codes)[u];
    const float sc = e8m0_to_f32(scales[u]);
    u32x4 *o = (u32x4 *)(out + (size_t)u * 32);
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = fp4x8_scaled_bf16_bits(wv[d], sc);
}

}  // namespace

moe_status mx_quantize_launch(int rows, int cols, const void *x, bool f32, uint8_t *codes, uint8_t *scales,
                              hipStream_t stream) {
    const long long nblk = (long long)rows * (cols / 32);
    if (nblk == 0) return MOE_OK;
    const int grid = (int)((nblk + 255) / 256);
    if (f32)
        hipLaunchKernelGGL(mx_quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, x, rows, cols, codes, scales);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, x, rows, cols, codes, scales);
    return launch_check("mx_quantize_kernel");
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_mx_quantize(int32_t rows, int32_t cols, const void *x, int32_t x_dtype,
                                      uint8_t *codes, uint8_t *scales, moe_stream stream) {
    clear_error();
    MOE_REQUIRE(rows >= 0 && cols > 0 && cols % 32 == 0,
                "moe_mx_quantize: need rows >= 0 and cols a positive multiple of 32 (rows=%d cols=%d)", rows, cols);
    MOE_REQUIRE(x_dtype == MOE_DT_BF16 || x_dtype == MOE_DT_F32, "moe_mx_quantize: unknown x_dtype %d", x_dtype);
    MOE_REQUIRE((int64_t)rows * cols < INT32_MAX, "moe_mx_quantize: sizes overflow int32");
    if (rows == 0) return MOE_OK;
    MOE_REQUIRE(x && codes && scales, "moe_mx_quantize: NULL pointer argument");
    return mx_quantize_launch(rows, cols, x, x_dtype == MOE_DT_F32, codes, scales, (hipStream_t)stream);
}

extern "C" moe_status moe_dequant(int32_t format, int32_t n, int32_t kdim, const uint8_t *codes,
                                  const void *scales, float *out, moe_stream stream) {
    clear_error();
    MOE_REQUIRE(format == MOE_W_MXFP4 || format == MOE_W_FP8_E4M3_B128, "moe_dequant: unknown format %d", format);
    MOE_REQUIRE(n >= 0 && kdim > 0, "moe_dequant: need n >= 0, kdim > 0");
    if (format == MOE_W_MXFP4)
        MOE_REQUIRE(kdim % 32 == 0, "moe_dequant: MXFP4 kdim = %d is not a multiple of 32", kdim);
    else
        MOE_REQUIRE(kdim % 128 == 0 && n % 128 == 0, "moe_dequant: FP8 n = %d and kdim = %d must be multiples of 128",
                    n, kdim);
    MOE_REQUIRE((int64_t)n * kdim < INT32_MAX, "moe_dequant: sizes overflow int32");
    if (n == 0) return MOE_OK;
    MOE_REQUIRE(codes && scales && out, "moe_dequant: NULL pointer argument");
    const long long units = (long long)n * (format == MOE_W_MXFP4 ? kdim / 32 : kdim / 16);
    const int grid = (int)((units + 255) / 256);
    hipStream_t s = (hipStream_t)stream;
    if (format == MOE_W_MXFP4)
        hipLaunchKernelGGL(dequant_kernel<0>, dim3(grid), dim3(256), 0, s, codes, scales, n, kdim, out);
    else
        hipLaunchKernelGGL(dequant_kernel<1>, dim3(grid), dim3(256), 0, s, codes, scales, n, kdim, out);
    return launch_check("moe_dequant");
}

extern "C" moe_status moe_dequant_bf16(int32_t n, int32_t kdim, const uint8_t *codes, const uint8_t *scales,
                                       uint16_t *out, moe_stream stream) {
    clear_error();
    MOE_REQUIRE(n >= 0 && kdim > 0 && kdim % 32 == 0,
                "moe_dequant_bf16: need n >= 0 and kdim a positive multiple of 32 (n=%d kdim=%d)", n, kdim);
    MOE_REQUIRE((int64_t)n * kdim < INT32_MAX, "moe_dequant_bf16: sizes overflow int32");
    if (n == 0) return MOE_OK;
    MOE_REQUIRE(codes && scales && out, "moe_dequant_bf16: NULL pointer argument");
    MOE_REQUIRE((((uintptr_t)codes | (uintptr_t)out) & 15) == 0, "moe_dequant_bf16: codes and out must be 16-byte aligned");
    const long long units = (long long)n * (kdim / 32);
    hipLaunchKernelGGL(dequant_bf16_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       codes, scales, units, out);
    return launch_check("moe_dequant_bf16");
}

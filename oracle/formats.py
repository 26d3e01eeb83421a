"""Number formats of the layer, decoded to exact float64 values.

The pages name the formats but print no tables: experts are stored as "OCP MXFP4" and
read as stored, with no conversion step (rabbit README, opening section and the
architecture table row "native quantization read"; Kimi K3 article, architecture
section), and GLM-5.2's experts as "FP8 (E4M3, block-scale)" (same tables).  The bit
layouts below are the ones the OCP Microscaling Formats (MX) v1.0 specification and
the OCP 8-bit floating point specification define for those names:

* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is subnormal
  (value = mantissa * 0.5).  No infinities or NaNs.
* E8M0 (the MX block scale): unsigned 8-bit exponent, value 2^(b-127); b = 255 is NaN.
* An MXFP4 block is 32 elements along the reduction axis sharing one E8M0 scale:
  16 code bytes + 1 scale byte, 17/32 byte per weight.  The rabbit README's 27 MB per
  expert and 24.6 GB per token agree with exactly that density.
* E4M3 ("FN" variant): sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at
  exponent 0, no infinities, S.1111.111 is NaN; largest finite 448.

Readings taken where the pages are silent: codes are stored row-major [N][K/2] with
the LOW nibble holding the even k; scales are [N][K/32]; FP8 block scales are float32
per 128x128 tile of the [N][K] matrix.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code):
    """Exact value of 4-bit E2M1 codes (array of ints 0..15) from the bit fields."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return sign * mag


def e8m0_value(b):
    """Exact value of E8M0 scale bytes: 2^(b-127), NaN for 0xFF."""
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def e4m3fn_value(b):
    """Exact value of E4M3 (FN) bytes."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((e == 15) & ((b & 7) == 7), np.nan, sign * mag)


def bf16_value(bits):
    """Exact value of bf16 bit patterns (uint16): the upper half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


_E2M1_BY_CODE = e2m1_value(np.arange(16))


def unpack_nibbles(codes):
    """[..., K/2] bytes -> [..., K] codes, element 2j from the low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def pack_nibbles(q):
    """Inverse of unpack_nibbles."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def dequant_mxfp4(codes, scales):
    """MXFP4 matrix -> float64 [N][K]: W[n][k] = E2M1(code[n][k]) * 2^(scale[n][k/32]-127)."""
    q = unpack_nibbles(codes)
    N, K = q.shape
    assert scales.shape == (N, K // 32), (scales.shape, (N, K // 32))
    return _E2M1_BY_CODE[q] * np.repeat(e8m0_value(scales), 32, axis=1)


def dequant_fp8_b128(codes, scales):
    """FP8 E4M3 matrix with one float32 scale per 128x128 tile -> float64 [N][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    assert scales.shape == (N // 128, K // 128)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), 128, axis=0), 128, axis=1)
    return e4m3fn_value(codes) * s


def dequant(fmt: str, codes, scales):
    return dequant_mxfp4(codes, scales) if fmt == "mxfp4" else dequant_fp8_b128(codes, scales)


_E2M1_MAGS = e2m1_value(np.arange(8))           # 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)
_EVEN_FIRST = [0, 2, 4, 6, 1, 3, 5, 7]


def mx_quantize(v):
    """OCP MX conversion of rows of values to MXFP4 codes and E8M0 scales, per 32-block.

    The pages only say the activations meet block-scaled FP4 weights; the conversion is
    the one the OCP MX v1.0 specification gives for a block of k = 32 values:
      1. shared exponent X = floor(log2(max |v|)) - emax, emax = 2 for E2M1, kept within
         the E8M0 range [-127, 127]; scale byte = X + 127;
      2. each element v / 2^X rounds to the nearest E2M1 value, ties to the code with an
         even mantissa bit, magnitudes above 6 saturate to 6; the sign is kept (so a
         negative value that rounds to zero gives -0).
    Readings: a block whose maximum is 0 gets scale byte 0 and zero codes; a block that
    holds a NaN or an infinity gets scale byte 0xFF and zero codes.
    Returns (codes [R][K/2] uint8, scales [R][K/32] uint8).
    """
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    assert K % 32 == 0
    blocks = v.reshape(R, K // 32, 32)
    bad = ~np.isfinite(blocks).all(axis=2)
    amax = np.where(bad, 0.0, np.abs(np.where(np.isfinite(blocks), blocks, 0.0)).max(axis=2))
    _, e = np.frexp(amax)                       # amax = m * 2^e, m in [0.5, 1)  ->  floor(log2 amax) = e - 1
    X = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    scaled = np.abs(np.where(np.isfinite(blocks), blocks, 0.0)) / np.exp2(X.astype(np.float64))[..., None]
    best = np.zeros(scaled.shape, dtype=np.int64)
    bestd = np.full(scaled.shape, np.inf)
    for j in _EVEN_FIRST:                        # strict '<' keeps the even code on a tie
        d = np.abs(scaled - _E2M1_MAGS[j])
        take = d < bestd
        best = np.where(take, j, best)
        bestd = np.where(take, d, bestd)
    sign = np.signbit(blocks).astype(np.int64) << 3
    q = (best | sign)
    q = np.where(bad[..., None], 0, q).astype(np.uint8).reshape(R, K)
    scales = np.where(bad, 255, X + 127).astype(np.uint8)
    return pack_nibbles(q), scales


def mx_dequantize(codes, scales):
    """Values of MX-quantised rows (the same decode as the weights)."""
    return dequant_mxfp4(codes, scales)

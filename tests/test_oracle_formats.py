"""Pins for oracle.formats against things other than the oracle itself.

Each format decoder is checked against either a hand-written table (tests/golden),
a library conversion (torch's float8_e4m3fn, float8_e8m0fnu and bfloat16 dtypes), or an
exhaustive brute force written with exact rational arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    assert sorted(vals) == list(range(16))
    return vals


def test_e2m1_matches_hand_table():
    g = _e2m1_golden()
    got = F.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == g[c], c
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, g[c]), c   # -0 for 0x8


def test_e8m0_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    got = F.e8m0_value(b)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e4m3_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3fn_value(b)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_bf16_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = F.bf16_value(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_nibble_order_hand_example():
    # byte 0x71: low nibble 0x1 (0.5) is element 0, high nibble 0x7 (6.0) is element 1.
    codes = np.full((1, 16), 0x71, np.uint8)
    codes[0, 1] = 0xA3          # elements 2, 3 = 1.5, -1.0
    W = F.dequant_mxfp4(codes, np.array([[127]], np.uint8))
    assert W[0, 0] == 0.5 and W[0, 1] == 6.0 and W[0, 2] == 1.5 and W[0, 3] == -1.0


def test_dequant_all_codes_times_all_scales():
    g = _e2m1_golden()
    # row b uses scale byte b; its 32 elements run through codes 0..15 twice
    q = np.tile(np.arange(16, dtype=np.uint8), 2)
    codes = np.tile(F.pack_nibbles(q)[None, :], (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    W = F.dequant_mxfp4(codes, scales)
    s_ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for b in range(256):
        for kk in range(32):
            want = g[kk % 16] * s_ref[b]
            if b == 255:
                assert np.isnan(W[b, kk])
            else:
                assert W[b, kk] == want, (b, kk)


def test_dequant_mxfp4_block_axis():
    rng = np.random.default_rng(1)
    N, K = 3, 96
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    W = F.dequant_mxfp4(codes, scales)
    g = _e2m1_golden()
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            assert W[n, k] == g[c] * 2.0 ** (int(scales[n, k // 32]) - 127)


def test_dequant_fp8_tile_scales():
    rng = np.random.default_rng(2)
    N, K = 256, 384
    codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    scales = np.ldexp(np.ones((2, 3), np.float32), rng.integers(-8, -3, (2, 3))).astype(np.float32)
    W = F.dequant_fp8_b128(codes, scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for n in range(0, N, 37):
        for k in range(0, K, 29):
            assert W[n, k] == ref[n, k] * float(scales[n // 128, k // 128])


def _read_mx_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "mx_quant_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        ent, sc, cd = [p.strip() for p in line.split("|")]
        entries = [(int(a), float(b)) for a, b in (e.split(":") for e in ent.split())] if ent else []
        codes = [int(c, 16) for c in cd.split()] if cd else []
        cases.append((entries, int(sc), codes))
    return cases


@pytest.mark.parametrize("case", _read_mx_cases())
def test_mx_quantize_hand_cases(case):
    entries, scale, codes = case
    v = np.zeros((1, 32))
    for i, x in entries:
        v[0, i] = x
    q, s = F.mx_quantize(v)
    assert int(s[0, 0]) == scale
    qq = F.unpack_nibbles(q)[0]
    want = np.zeros(32, np.int64)
    for (i, _), c in zip(entries, codes):
        want[i] = c
    np.testing.assert_array_equal(qq, want)


def _rne_e2m1_exact(a: Fraction) -> int:
    """Brute-force reference: bracket |a| between consecutive E2M1 magnitudes, pick the
    nearer, on an exact tie the one whose code is even; beyond 6 -> 6."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    if a >= 6:
        return 7
    for c in range(7):
        lo, hi = mags[c], mags[c + 1]
        if lo <= a <= hi:
            dl, dh = a - lo, hi - a
            if dl < dh:
                return c
            if dh < dl:
                return c + 1
            return c if c % 2 == 0 else c + 1
    raise AssertionError


def test_mx_quantize_exhaustive_bf16_against_exact_rounding():
    # every finite bf16 value v, placed in a block whose max magnitude is 6 * 2^3 (X = 3),
    # must round like the exact-rational brute force of v / 8.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_value(bits)
    ok = np.isfinite(vals) & (np.abs(vals) <= 48.0)
    vals = vals[ok]
    n = len(vals)
    blocks = np.zeros((n, 32))
    blocks[:, 0] = 48.0
    blocks[:, 1] = vals
    q, s = F.mx_quantize(blocks)
    assert (s == 130).all()
    got = F.unpack_nibbles(q)[:, 1]
    for v, c in zip(vals, got):
        mag = _rne_e2m1_exact(abs(Fraction(float(v))) / 8)
        want = mag | (8 if math.copysign(1.0, v) < 0 else 0)
        assert c == want, (v, c, want)


def test_mx_quantize_scale_byte_rule():
    for amax, want in [(1.0, 125), (1.999, 125), (2.0, 126), (6.0, 127), (8.0, 128), (0.75, 124),
                       (2.0 ** -125, 0), (2.0 ** -130, 0), (0.0, 0), (3e38, 127 + 127 - 2)]:
        v = np.zeros((1, 32))
        v[0, 3] = amax
        _, s = F.mx_quantize(v)
        assert int(s[0, 0]) == want, (amax, int(s[0, 0]), want)
    v = np.zeros((1, 64))
    v[0, 40] = np.nan
    q, s = F.mx_quantize(v)
    assert list(s[0]) == [0, 255]


def test_mx_roundtrip_of_representable_values():
    g = _e2m1_golden()
    rng = np.random.default_rng(3)
    for X in (-10, -2, 0, 5):
        codes = rng.integers(0, 16, (4, 32))
        codes[:, 0] = 7      # each block reaches 6 * 2^X, so the scale is 2^X
        v = np.vectorize(lambda c: g[int(c)])(codes) * 2.0 ** X
        q, s = F.mx_quantize(v)
        assert (s == X + 127).all()
        np.testing.assert_array_equal(F.mx_dequantize(q, s), v)
        # quantising a second time changes nothing (idempotent)
        q2, s2 = F.mx_quantize(F.mx_dequantize(q, s))
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s)

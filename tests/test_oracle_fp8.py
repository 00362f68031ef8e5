"""Pins for the e4m3 quantizer of the oracle (CPU only): code values from the
format's definition, ties to even, saturation, the sign of zero, the round trip
of every code, and nearest rounding checked by brute force over the code table."""

import numpy as np
import pytest

from oracle import fp8 as F


@pytest.mark.parametrize("x,code", [
    (0.0, 0x00), (-0.0, 0x80), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08),
    (0.5, 0x30), (1.0, 0x38), (1.5, 0x3C), (-1.5, 0xBC), (240.0, 0x77), (256.0, 0x78),
    (448.0, 0x7E), (-448.0, 0xFE),
])
def test_known_codes(x, code):
    assert F.quantize_e4m3(np.float32(x)) == code
    assert F.dequantize_e4m3(np.uint8(code)) == x or (x == 0 and F.dequantize_e4m3(np.uint8(code)) == 0)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),           # halfway 1.0 (0x38) .. 1.125 (0x39): the even code
    (1.1875, 0x3A),           # halfway 1.125 (0x39) .. 1.25 (0x3A)
    (3 * 2.0 ** -10, 0x02),   # halfway between subnormals 1 and 2
    (2.0 ** -10, 0x00),       # halfway between 0 and the smallest subnormal
    (-2.0 ** -10, 0x80),
    (464.0, 0x7E),            # beyond 448: saturates (no infinity in e4m3)
    (1e30, 0x7E), (-1e30, 0xFE),
])
def test_ties_to_even_and_saturation(x, code):
    assert F.quantize_e4m3(np.float32(x)) == code


def test_value_table_is_the_format():
    v = F.e4m3_positive_values()
    assert v[0] == 0 and v[1] == 2.0 ** -9 and v[126] == 448.0
    assert np.all(np.diff(v) > 0)                       # strictly increasing
    for E in range(1, 16):
        for m in range(8):
            c = (E << 3) | m
            if c < 127:
                assert v[c] == (8 + m) * 2.0 ** (E - 10)


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = F.dequantize_e4m3(codes)
    back = F.quantize_e4m3(vals.astype(np.float32))
    # -0.0 keeps its sign: 0x80 round trips to 0x80
    assert np.array_equal(back, codes)


def test_nearest_by_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x.astype(np.float32)
    q = F.quantize_e4m3(x)
    got = F.dequantize_e4m3(q)
    table = np.concatenate([-F.e4m3_positive_values(), F.e4m3_positive_values()])
    for xi, gi in zip(x.astype(np.float64), got):
        best = np.min(np.abs(table - xi))
        assert abs(gi - xi) == best


def test_scale_divides_before_rounding():
    # 1.0 / 0.75 = 1.333..: between 1.25 (0x3A) and 1.375 (0x3B), nearer 1.375
    assert F.quantize_e4m3(np.float32(1.0), np.float32(1.0) / np.float32(0.75)) == 0x3B
    assert F.dequantize_e4m3(np.uint8(0x3B), 0.75) == 1.375 * 0.75


@pytest.mark.parametrize("bits,inv,code", [
    (0x3F80, 1.0, 0x38),          # 1.0
    (0x3FC0, 1.0, 0x3C),          # 1.5
    (0xBFC0, 1.0, 0xBC),          # -1.5
    (0x43E0, 1.0, 0x7E),          # 448, the largest e4m3 value
    (0x4400, 1.0, 0x7E),          # 512 saturates
    (0xC400, 1.0, 0xFE),          # -512 saturates
    (0x8000, 1.0, 0x80),          # -0 keeps its sign
    (0x0000, 1.0, 0x00),
    (0x0001, 1.0, 0x00),          # a bf16 subnormal (~9e-41) rounds to zero
    (0x8001, 1.0, 0x80),          # ... and its negative to -0
    (0x3F88, 1.0, 0x38),          # 1.0625: halfway 1.0 .. 1.125, the even code
    (0x3F98, 1.0, 0x3A),          # 1.1875: halfway 1.125 .. 1.25, the even code
    (0x3B40, 1.0, 0x02),          # 3 * 2^-10: halfway between subnormal codes 1 and 2
    (0x3B00, 1.0, 0x01),          # 2^-9, the smallest subnormal
    (0x3A80, 1.0, 0x00),          # 2^-10: halfway 0 .. 2^-9, the even code 0
    (0x3F80, 1.0 / 0.75, 0x3B),   # 1 / 0.75 = 1.333..: nearest 1.375
    (0x4040, 0.5, 0x3C),          # 3 * 0.5 = 1.5
    (0x4396, 2.0, 0x7E),          # 300 * 2 = 600 saturates
    (0x3C00, 64.0, 0x30),         # 2^-7 * 64 = 0.5
])
def test_bf16_bits_to_codes(bits, inv, code):
    """The stored form of a bf16 K/V value, from its bit pattern: expected codes
    follow from the two formats' definitions (bf16: 1 sign, 8 exponent bits of bias
    127, 7 mantissa bits; e4m3 as above)."""
    got = F.bf16_to_e4m3(np.array([bits], dtype=np.uint16), np.float32(inv))
    assert got.dtype == np.uint8 and got.shape == (1,)
    assert int(got[0]) == code


def _bf16_value(bits: int) -> float:
    """bf16 bit pattern -> value, decoded field by field (no float reinterpretation)."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    mag = m * 2.0 ** -133 if e == 0 else (1 + m / 128.0) * 2.0 ** (e - 127)
    return -mag if s else mag


def test_bf16_bits_every_finite_pattern():
    """All 65,280 finite bf16 patterns at once: the codes equal the quantizer applied
    to values decoded field by field, and each code is a nearest e4m3 value to its
    input clamped to +-448 (a wrong shift or widening fails this)."""
    bits = np.array([b for b in range(1 << 16) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    vals = np.array([_bf16_value(int(b)) for b in bits])
    codes = F.bf16_to_e4m3(bits)
    assert np.array_equal(codes, F.quantize_e4m3(vals.astype(np.float32)))
    back = F.dequantize_e4m3(codes)
    clamped = np.clip(vals, -448.0, 448.0)
    table = np.concatenate([-F.e4m3_positive_values(), F.e4m3_positive_values()])
    nearest = np.min(np.abs(clamped[:, None] - table[None, :]), axis=1)
    assert np.array_equal(np.abs(back - clamped), nearest)
    assert np.array_equal(np.signbit(back) | (back == 0), np.signbit(vals) | (back == 0))

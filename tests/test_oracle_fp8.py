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

"""Pins of the oracle's weight decoding against hand-built bytes.

Every expected value here is written by hand from the format definitions
(fp16 scale first, GGUF nibble order for Q4_0 and Q4_1, Q4_1's fp16 minimum
after the scale, low nibble = even weight and two's complement for packed
int4, low bit pair first and two's complement for packed int2), never
computed by the oracle."""
import os

import numpy as np
import pytest

from synth import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp16_values.txt")


def _fp16_table():
    rows = []
    with open(GOLD) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            h, v = line.split()
            rows.append((int(h, 16), float(v)))
    return rows


@pytest.mark.parametrize("bits,value", _fp16_table())
def test_q8_0_scale_is_ieee_binary16(orc, bits, value):
    # one block, all q = 1: every weight equals d exactly
    blk = bytes([bits & 0xFF, bits >> 8]) + bytes([1] * 32)
    w = orc.decode_row("q8_0", blk, 0.0, 32)
    assert np.all(w == value)
    assert np.all(np.signbit(w) == np.signbit(value))


def test_q8_0_ramp_and_sign(orc):
    q = bytes(range(0, 32))                      # 0..31
    w = orc.decode_row("q8_0", bytes([0x00, 0x3C]) + q, 0.0, 32)
    assert list(w) == list(range(32))
    q = bytes([0x80, 0xFF, 0x7F, 0x01] + [0] * 28)   # -128, -1, 127, 1
    w = orc.decode_row("q8_0", bytes([0x00, 0xC0]) + q, 0.0, 32)   # d = -2
    assert list(w[:4]) == [256.0, 2.0, -254.0, -2.0]
    assert np.all(w[4:] == 0)


def test_q8_0_two_blocks_use_their_own_scale(orc):
    row = bytes([0x00, 0x3C]) + bytes([3] * 32) + bytes([0x00, 0x38]) + bytes([3] * 32)
    w = orc.decode_row("q8_0", row, 0.0, 64)
    assert np.all(w[:32] == 3.0) and np.all(w[32:] == 1.5)


def test_q8_0_zero_and_subnormal_scale(orc):
    w = orc.decode_row("q8_0", bytes([0, 0]) + bytes([0x7F] * 32), 0.0, 32)
    assert np.all(w == 0.0)
    w = orc.decode_row("q8_0", bytes([1, 0]) + bytes([0x7F] * 32), 0.0, 32)
    assert np.all(w == 127 * 2.0 ** -24)


@pytest.mark.parametrize("j", [0, 5, 15])
def test_q4_0_nibble_order(orc, j):
    # all nibbles 8 (weight 0) except the low nibble of byte j -> weight j,
    # or the high nibble of byte j -> weight j + 16
    qs = bytearray([0x88] * 16)
    qs[j] = 0x8B                                  # low nibble 11 -> +3
    w = orc.decode_row("q4_0", bytes([0x00, 0x3C]) + bytes(qs), 0.0, 32)
    exp = np.zeros(32)
    exp[j] = 3.0
    assert np.array_equal(w, exp)
    qs = bytearray([0x88] * 16)
    qs[j] = 0x28                                  # high nibble 2 -> -6
    w = orc.decode_row("q4_0", bytes([0x00, 0x40]) + bytes(qs), 0.0, 32)   # d = 2
    exp = np.zeros(32)
    exp[j + 16] = -12.0
    assert np.array_equal(w, exp)


def test_q4_0_extremes(orc):
    w = orc.decode_row("q4_0", bytes([0x00, 0x3C]) + bytes([0x0F] * 16), 0.0, 32)
    assert np.all(w[:16] == 7.0) and np.all(w[16:] == -8.0)


def test_i8_row(orc):
    row = bytes([0x80, 0xFF, 0x00, 0x7F, 0x02])
    w = orc.decode_row("i8_row", row + bytes(11), 0.5, 16)
    assert list(w[:5]) == [-64.0, -0.5, 0.0, 63.5, 1.0]


def test_i4_row_order_and_sign(orc):
    # byte 0x8F: weight 0 = nibble 0xF = -1, weight 1 = nibble 0x8 = -8
    # byte 0x70: weight 2 = 0, weight 3 = 7;  byte 0x21: weight 4 = 1, weight 5 = 2
    w = orc.decode_row("i4_row", bytes([0x8F, 0x70, 0x21, 0x00]), 0.25, 8)
    assert list(w) == [-0.25, -2.0, 0.0, 1.75, 0.25, 0.5, 0.0, 0.0]


def test_i4_row_scale_product_is_exact(orc):
    s = np.float32(0.0012345678)
    w = orc.decode_row("i4_row", bytes([0x77]), float(s), 2)
    assert w[0] == 7.0 * float(s) and w[1] == 7.0 * float(s)


def test_q4_1_nibble_order_and_minimum(orc):
    # d = 0.5 (0x3800), m = 0.25 (0x3400): w = 0.5 n + 0.25; byte 5 = 0x3A gives
    # weight 5 the low nibble 10 and weight 21 the high nibble 3
    qs = bytearray(16)
    qs[5] = 0x3A
    w = orc.decode_row("q4_1", bytes([0x00, 0x38, 0x00, 0x34]) + bytes(qs), 0.0, 32)
    exp = np.full(32, 0.25)
    exp[5] = 5.25
    exp[21] = 1.75
    assert np.array_equal(w, exp)


def test_q4_1_extremes_and_second_block(orc):
    # block 0: d = 1, m = -8 (0xC800), all codes 15 -> 7; block 1: d = 2
    # (0x4000), m = 0, all codes 0 -> 0
    row = bytes([0x00, 0x3C, 0x00, 0xC8]) + bytes([0xFF] * 16) + bytes([0x00, 0x40, 0x00, 0x00]) + bytes(16)
    w = orc.decode_row("q4_1", row, 0.0, 64)
    assert np.all(w[:32] == 7.0) and np.all(w[32:] == 0.0)


def test_q4_1_sum_is_exact(orc):
    # d = 2^-24 (smallest subnormal, 0x0001), m = 1024 (0x6400), codes 15:
    # w = 1024 + 15 * 2^-24 exactly (fp32 could not hold it)
    w = orc.decode_row("q4_1", bytes([0x01, 0x00, 0x00, 0x64]) + bytes([0xFF] * 16), 0.0, 32)
    assert np.all(w - 1024.0 == 15 * 2.0 ** -24)


def test_i2_row_order_and_sign(orc):
    # byte 0xE4 = 0b11_10_01_00: weights 0..3 = 0, 1, -2, -1;
    # byte 0x1B = 0b00_01_10_11: weights 4..7 = -1, -2, 1, 0
    w = orc.decode_row("i2_row", bytes([0xE4, 0x1B, 0x00, 0xFF]), 0.5, 16)
    assert list(w) == [0.0, 0.5, -1.0, -0.5, -0.5, -1.0, 0.5, 0.0, 0.0, 0.0, 0.0, 0.0, -0.5, -0.5, -0.5, -0.5]


def test_row_bytes(orc):
    assert orc.row_bytes("q8_0", 256) == 272 == F.row_bytes("q8_0", 256)
    assert orc.row_bytes("q4_0", 768) == 432 == F.row_bytes("q4_0", 768)
    assert orc.row_bytes("i8_row", 2048) == 2048 == F.row_bytes("i8_row", 2048)
    assert orc.row_bytes("i4_row", 6144) == 3072 == F.row_bytes("i4_row", 6144)
    assert orc.row_bytes("q4_1", 2560) == 1600 == F.row_bytes("q4_1", 2560)
    assert orc.row_bytes("i2_row", 6144) == 1536 == F.row_bytes("i2_row", 6144)
    assert orc.row_bytes("q8_0", 33) == -1
    assert orc.row_bytes("i2_row", 6) == -1


# ---- the generator's packers, checked through the (now pinned) decoder ----

def test_packers_round_trip(orc):
    rng = np.random.default_rng(7)
    rows, cols = 3, 64
    d = rng.uniform(1e-3, 1e-2, (rows, 2)).astype(np.float16)
    q = rng.integers(-128, 128, (rows, cols))
    m = F.pack_q8_0(d, q)
    for r in range(rows):
        w = orc.decode_row("q8_0", m.data[r], 0.0, cols)
        exp = np.repeat(d[r].astype(np.float64), 32) * q[r]
        assert np.array_equal(w, exp)
    n = rng.integers(0, 16, (rows, cols))
    m = F.pack_q4_0(d, n)
    for r in range(rows):
        w = orc.decode_row("q4_0", m.data[r], 0.0, cols)
        assert np.array_equal(w, np.repeat(d[r].astype(np.float64), 32) * (n[r] - 8))
    s = rng.uniform(1e-3, 1e-2, rows).astype(np.float32)
    v = rng.integers(-8, 8, (rows, cols))
    m = F.pack_i4_row(s, v)
    for r in range(rows):
        w = orc.decode_row("i4_row", m.data[r], float(m.scales[r]), cols)
        assert np.array_equal(w, float(s[r]) * v[r])
    m = F.pack_i8_row(s, q)
    for r in range(rows):
        w = orc.decode_row("i8_row", m.data[r], float(m.scales[r]), cols)
        assert np.array_equal(w, float(s[r]) * q[r])
    mn = (-d.astype(np.float64) * 7).astype(np.float16)
    m = F.pack_q4_1(d, mn, n)
    for r in range(rows):
        w = orc.decode_row("q4_1", m.data[r], 0.0, cols)
        exp = np.repeat(d[r].astype(np.float64), 32) * n[r] + np.repeat(mn[r].astype(np.float64), 32)
        assert np.array_equal(w, exp)
    v2 = rng.integers(-2, 2, (rows, cols))
    m = F.pack_i2_row(s, v2)
    for r in range(rows):
        w = orc.decode_row("i2_row", m.data[r], float(m.scales[r]), cols)
        assert np.array_equal(w, float(s[r]) * v2[r])


def test_bf16_rounding_of_inputs():
    x = np.array([1.0, 1.00390625, 1.0 + 2 ** -8 + 2 ** -9, -3.0, 0.0], dtype=np.float32)
    b = F.f32_to_bf16_bits(x)
    assert list(b) == [0x3F80, 0x3F80, 0x3F81, 0xC040, 0x0000]

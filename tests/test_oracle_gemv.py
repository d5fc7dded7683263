"""Pins of the oracle's quantized GEMV: closed forms, one-hot columns, a
float64 library matmul on independently built weights, and invariants."""
import numpy as np
import pytest

from synth import formats as F


def _fp32_ok(y, exact, S, rel=1e-12):
    """y is exact rounded to fp32, up to double summation-order noise."""
    exact = np.asarray(exact, dtype=np.float64)
    return np.all(np.abs(y.astype(np.float64) - exact) <= np.abs(exact) * 2.0 ** -24 + rel * S + 1e-300)


def _x(rng, B, K):
    return rng.standard_normal((B, K)).astype(np.float32)


def test_q8_0_all_ones_closed_form(orc):
    rng = np.random.default_rng(1)
    rows, K = 5, 96
    d = rng.uniform(1e-3, 1e-2, (rows, 3)).astype(np.float16)
    m = F.pack_q8_0(d, np.ones((rows, K), dtype=np.int64))
    x = _x(rng, 1, K)
    y, S = orc.qgemv(m, x)
    bs = x[0].astype(np.float64).reshape(3, 32).sum(axis=1)      # per-block sum of x
    exact = (d.astype(np.float64) * bs[None, :]).sum(axis=1)
    assert _fp32_ok(y[0], exact, S[0])
    assert np.allclose(S[0], (d.astype(np.float64) * np.abs(x[0]).astype(np.float64).reshape(3, 32).sum(1)).sum(1))


def test_q4_0_nine_is_one_and_eight_is_zero(orc):
    rng = np.random.default_rng(2)
    rows, K = 4, 64
    d = rng.uniform(1e-3, 2e-2, (rows, 2)).astype(np.float16)
    x = _x(rng, 2, K)
    y, S = orc.qgemv(F.pack_q4_0(d, np.full((rows, K), 9)), x)
    for b in range(2):
        exact = (d.astype(np.float64) * x[b].astype(np.float64).reshape(2, 32).sum(1)).sum(1)
        assert _fp32_ok(y[b], exact, S[b])
    y0, S0 = orc.qgemv(F.pack_q4_0(d, np.full((rows, K), 8)), x)
    assert np.all(y0 == 0.0) and np.all(S0 == 0.0)


def test_q4_1_code_times_d_cancels_minimum(orc):
    # codes all 4 and m = -4 d: every weight is exactly zero; codes all 0:
    # y = sum over blocks of m times the block's sum of x
    rng = np.random.default_rng(8)
    rows, K = 5, 96
    d = rng.uniform(1e-3, 2e-2, (rows, 3)).astype(np.float16)
    mn = (-4 * d.astype(np.float64)).astype(np.float16)      # exact: a power-of-two multiple
    assert np.array_equal(mn.astype(np.float64), -4 * d.astype(np.float64))
    x = _x(rng, 2, K)
    y, S = orc.qgemv(F.pack_q4_1(d, mn, np.full((rows, K), 4)), x)
    assert np.all(y == 0.0) and np.all(S == 0.0)
    y, S = orc.qgemv(F.pack_q4_1(d, mn, np.zeros((rows, K), dtype=np.int64)), x)
    for b in range(2):
        exact = (mn.astype(np.float64) * x[b].astype(np.float64).reshape(3, 32).sum(1)).sum(1)
        assert _fp32_ok(y[b], exact, S[b])


def test_i2_row_alternating_signs(orc):
    # weights +1, -1, +1, -1, ... (codes 1, 3): y = s * (x0 - x1 + x2 - x3 ...)
    s = np.array([0.25, 0.003], dtype=np.float32)
    v = np.tile([1, -1], (2, 128))
    rng = np.random.default_rng(9)
    x = _x(rng, 1, 256)
    y, S = orc.qgemv(F.pack_i2_row(s, v), x)
    alt = x[0].astype(np.float64)[0::2].sum() - x[0].astype(np.float64)[1::2].sum()
    assert _fp32_ok(y[0], s.astype(np.float64) * alt, S[0])


def test_i8_row_ones_times_ones(orc):
    s = np.array([0.5, 0.001, 0.0037], dtype=np.float32)
    m = F.pack_i8_row(s, np.ones((3, 256), dtype=np.int64))
    y, _ = orc.qgemv(m, np.ones((1, 256), dtype=np.float32))
    assert np.array_equal(y[0], (s.astype(np.float64) * 256).astype(np.float32))


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_one_hot_x_reads_one_weight(orc, fmt):
    rng = np.random.default_rng(3)
    rows, K = 6, 64
    m, W = _random_matrix(rng, fmt, rows, K)
    for c in (0, 17, 63):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, c] = 1.0
        y, _ = orc.qgemv(m, x)
        assert np.array_equal(y[0], W[:, c].astype(np.float32))


def _random_matrix(rng, fmt, rows, K):
    """A random matrix built from integer codes and scales, together with its
    float64 values computed here from those codes (not by the oracle)."""
    if fmt == "q8_0":
        d = rng.uniform(1e-3, 1e-2, (rows, K // 32)).astype(np.float16)
        q = rng.integers(-127, 128, (rows, K))
        return F.pack_q8_0(d, q), np.repeat(d.astype(np.float64), 32, axis=1) * q
    if fmt == "q4_0":
        d = rng.uniform(1e-3, 2e-2, (rows, K // 32)).astype(np.float16)
        n = rng.integers(0, 16, (rows, K))
        return F.pack_q4_0(d, n), np.repeat(d.astype(np.float64), 32, axis=1) * (n - 8)
    if fmt == "q4_1":
        d = rng.uniform(1e-3, 2e-2, (rows, K // 32)).astype(np.float16)
        mn = rng.uniform(-0.2, 0.05, (rows, K // 32)).astype(np.float16)
        n = rng.integers(0, 16, (rows, K))
        return (F.pack_q4_1(d, mn, n),
                np.repeat(d.astype(np.float64), 32, axis=1) * n + np.repeat(mn.astype(np.float64), 32, axis=1))
    s = rng.uniform(1e-3, 1e-2, rows).astype(np.float32)
    if fmt == "i8_row":
        q = rng.integers(-127, 128, (rows, K))
        return F.pack_i8_row(s, q), s.astype(np.float64)[:, None] * q
    if fmt == "i2_row":
        v = rng.integers(-2, 2, (rows, K))
        return F.pack_i2_row(s, v), s.astype(np.float64)[:, None] * v
    assert fmt == "i4_row"
    v = rng.integers(-8, 8, (rows, K))
    return F.pack_i4_row(s, v), s.astype(np.float64)[:, None] * v


@pytest.mark.parametrize("fmt", F.FORMATS)
@pytest.mark.parametrize("shape", [(7, 256), (33, 512), (16, 2048)])
def test_matches_float64_matmul(orc, fmt, shape):
    rng = np.random.default_rng([F.FORMATS.index(fmt), shape[0], shape[1]])
    rows, K = shape
    m, W = _random_matrix(rng, fmt, rows, K)
    x = _x(rng, 3, K)
    y, S = orc.qgemv(m, x)
    ref = x.astype(np.float64) @ W.T                       # library matmul
    Sref = np.abs(x.astype(np.float64)) @ np.abs(W.T)
    assert np.allclose(S, Sref, rtol=1e-12, atol=0)
    assert _fp32_ok(y, ref, S)


def test_bf16_activations(orc):
    rng = np.random.default_rng(4)
    m, W = _random_matrix(rng, "q4_0", 9, 256)
    xb = F.f32_to_bf16_bits(rng.standard_normal((2, 256)))
    xf = (xb.astype(np.uint32) << 16).view(np.float32)     # bf16 is the top half of fp32
    yb, Sb = orc.qgemv(m, xb, "bf16")
    yf, Sf = orc.qgemv(m, xf, "f32")
    assert np.array_equal(yb, yf) and np.array_equal(Sb, Sf)


def test_batch_equals_single_calls_and_linearity(orc):
    rng = np.random.default_rng(5)
    m, _ = _random_matrix(rng, "q8_0", 12, 512)
    x = _x(rng, 4, 512)
    y, _ = orc.qgemv(m, x)
    for b in range(4):
        yb, _ = orc.qgemv(m, x[b:b + 1])
        assert np.array_equal(yb[0], y[b])
    # scaling x by a power of two scales y exactly
    y2, _ = orc.qgemv(m, x * 4.0)
    assert np.array_equal(y2, y * 4.0)


def test_threads_bitwise(orc, orc_mt):
    rng = np.random.default_rng(6)
    m, _ = _random_matrix(rng, "i4_row", 64, 1024)
    x = _x(rng, 2, 1024)
    y1, S1 = orc.qgemv(m, x)
    y2, S2 = orc_mt.qgemv(m, x)
    assert np.array_equal(y1, y2) and np.array_equal(S1, S2)

"""Canonical byte layouts of the four weight formats (layout only, no arithmetic).

A matrix has ``rows`` output rows of ``cols`` weights, stored row-major, one
row after another.  Formats (the block formats follow the GGUF convention that
the Camelid README's "Engine" and "Supported" sections name for its Q8_0 and
Q4_0 rows; the per-row formats are the int8 / packed-int4 per-row-scale
formats of the colibri summary, "model execution and memory tiers"):

``q8_0``    blocks of 32 weights, 34 bytes: fp16 scale d (little-endian), then
            32 signed bytes q[0..31].
``q4_0``    blocks of 32 weights, 18 bytes: fp16 scale d, then 16 bytes qs;
            weight j (0..15) is the low nibble of qs[j], weight j+16 its high
            nibble; nibbles are unsigned 0..15 and carry an offset of 8.
``i8_row``  ``cols`` signed bytes per row; one fp32 scale per row kept in a
            separate array.
``i4_row``  ``cols/2`` bytes per row; weight 2j is the low nibble of byte j,
            weight 2j+1 its high nibble; nibbles are two's-complement in
            [-8, 7]; one fp32 scale per row kept in a separate array.
``q4_1``    blocks of 32 weights, 20 bytes: fp16 scale d, fp16 minimum m, then
            16 bytes qs in the q4_0 nibble order; codes n in 0..15 carry no
            offset (the value is d * n + m).  The GGUF block the Camelid
            README names for its bit-exact q4_1 GEMV ("Experimental" rows).
``i2_row``  ``cols/4`` bytes per row; weight 4j+i sits in bits 2i..2i+1 of
            byte j as a two's-complement integer in [-2, 1]; one fp32 scale per
            row kept in a separate array (the packed int2 per-row format of
            the colibri summary, "model execution and memory tiers").
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

FORMATS = ("q8_0", "q4_0", "i8_row", "i4_row", "q4_1", "i2_row")
ROW_FORMATS = ("i8_row", "i4_row", "i2_row")
_BLOCK = 32


def blocks_per_row(fmt: str, cols: int) -> int:
    if fmt not in ("q8_0", "q4_0", "q4_1"):
        raise ValueError(f"{fmt} has no blocks")
    if cols % _BLOCK:
        raise ValueError("cols must be a multiple of 32")
    return cols // _BLOCK


def row_bytes(fmt: str, cols: int) -> int:
    """Bytes of one row in the canonical layout (row scales not included)."""
    if fmt == "q8_0":
        return blocks_per_row(fmt, cols) * 34
    if fmt == "q4_0":
        return blocks_per_row(fmt, cols) * 18
    if fmt == "i8_row":
        return cols
    if fmt == "i4_row":
        if cols % 2:
            raise ValueError("i4_row needs an even number of columns")
        return cols // 2
    if fmt == "q4_1":
        return blocks_per_row(fmt, cols) * 20
    if fmt == "i2_row":
        if cols % 4:
            raise ValueError("i2_row needs a multiple of 4 columns")
        return cols // 4
    raise ValueError(f"unknown format {fmt!r}")


def matrix_bytes(fmt: str, rows: int, cols: int) -> int:
    """Weight bytes of a matrix, including the per-row fp32 scales."""
    extra = 4 * rows if fmt in ROW_FORMATS else 0
    return rows * row_bytes(fmt, cols) + extra


@dataclass
class QMatrix:
    """A quantized matrix in the canonical layout.

    ``data``   uint8 array of shape (rows, row_bytes(fmt, cols)).
    ``scales`` float32 array of shape (rows,) for the per-row formats, else None.
    """
    fmt: str
    rows: int
    cols: int
    data: np.ndarray
    scales: Optional[np.ndarray] = None

    @property
    def nbytes(self) -> int:
        return matrix_bytes(self.fmt, self.rows, self.cols)


def _as_u16(d_bits) -> np.ndarray:
    d = np.asarray(d_bits)
    if d.dtype == np.float16:
        d = d.view(np.uint16)
    return d.astype(np.uint16)


def pack_q8_0(d_bits, q) -> QMatrix:
    """Lay out Q8_0 blocks.  ``d_bits``: (rows, cols/32) fp16 (or its uint16
    bits); ``q``: (rows, cols) integers in [-128, 127]."""
    q = np.asarray(q)
    rows, cols = q.shape
    nb = blocks_per_row("q8_0", cols)
    d = _as_u16(d_bits).reshape(rows, nb)
    out = np.empty((rows, nb, 34), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2:] = q.astype(np.int8).reshape(rows, nb, 32).view(np.uint8)
    return QMatrix("q8_0", rows, cols, out.reshape(rows, nb * 34))


def pack_q4_0(d_bits, n) -> QMatrix:
    """Lay out Q4_0 blocks.  ``n``: (rows, cols) unsigned nibbles 0..15
    (the stored code, before the offset of 8)."""
    n = np.asarray(n).astype(np.uint8)
    if n.max(initial=0) > 15:
        raise ValueError("q4_0 nibbles must be in 0..15")
    rows, cols = n.shape
    nb = blocks_per_row("q4_0", cols)
    d = _as_u16(d_bits).reshape(rows, nb)
    nn = n.reshape(rows, nb, 32)
    out = np.empty((rows, nb, 18), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2:] = nn[:, :, :16] | (nn[:, :, 16:] << 4)
    return QMatrix("q4_0", rows, cols, out.reshape(rows, nb * 18))


def pack_i8_row(scales, q) -> QMatrix:
    """Lay out int8 rows.  ``q``: (rows, cols) integers in [-128, 127]."""
    q = np.asarray(q)
    rows, cols = q.shape
    data = q.astype(np.int8).view(np.uint8).reshape(rows, cols).copy()
    return QMatrix("i8_row", rows, cols, data, np.asarray(scales, dtype=np.float32).reshape(rows))


def pack_i4_row(scales, v) -> QMatrix:
    """Lay out packed signed int4 rows.  ``v``: (rows, cols) integers in [-8, 7]."""
    v = np.asarray(v).astype(np.int16)
    if v.min(initial=0) < -8 or v.max(initial=0) > 7:
        raise ValueError("i4_row values must be in [-8, 7]")
    rows, cols = v.shape
    code = (v & 0xF).astype(np.uint8)            # two's-complement nibble
    data = code[:, 0::2] | (code[:, 1::2] << 4)
    return QMatrix("i4_row", rows, cols, np.ascontiguousarray(data),
                   np.asarray(scales, dtype=np.float32).reshape(rows))


def pack_q4_1(d_bits, m_bits, n) -> QMatrix:
    """Lay out Q4_1 blocks.  ``d_bits``, ``m_bits``: (rows, cols/32) fp16 (or
    their uint16 bits); ``n``: (rows, cols) unsigned codes 0..15."""
    n = np.asarray(n).astype(np.uint8)
    if n.max(initial=0) > 15:
        raise ValueError("q4_1 codes must be in 0..15")
    rows, cols = n.shape
    nb = blocks_per_row("q4_1", cols)
    d = _as_u16(d_bits).reshape(rows, nb)
    m = _as_u16(m_bits).reshape(rows, nb)
    nn = n.reshape(rows, nb, 32)
    out = np.empty((rows, nb, 20), dtype=np.uint8)
    out[:, :, 0] = (d & 0xFF).astype(np.uint8)
    out[:, :, 1] = (d >> 8).astype(np.uint8)
    out[:, :, 2] = (m & 0xFF).astype(np.uint8)
    out[:, :, 3] = (m >> 8).astype(np.uint8)
    out[:, :, 4:] = nn[:, :, :16] | (nn[:, :, 16:] << 4)
    return QMatrix("q4_1", rows, cols, out.reshape(rows, nb * 20))


def pack_i2_row(scales, v) -> QMatrix:
    """Lay out packed signed int2 rows.  ``v``: (rows, cols) integers in [-2, 1]."""
    v = np.asarray(v).astype(np.int16)
    if v.min(initial=0) < -2 or v.max(initial=0) > 1:
        raise ValueError("i2_row values must be in [-2, 1]")
    rows, cols = v.shape
    if cols % 4:
        raise ValueError("i2_row needs a multiple of 4 columns")
    code = (v & 3).astype(np.uint8)               # two's-complement 2-bit code
    data = code[:, 0::4] | (code[:, 1::4] << 2) | (code[:, 2::4] << 4) | (code[:, 3::4] << 6)
    return QMatrix("i2_row", rows, cols, np.ascontiguousarray(data),
                   np.asarray(scales, dtype=np.float32).reshape(rows))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Used to draw bf16 inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)

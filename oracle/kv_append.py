"""Oracle for writing new tokens into the paged KV pool (TEST INFRASTRUCTURE
ONLY: only the tests, the package smoke check and the benchmark's
CPU-baseline leg may use it; the product library never calls it).

The row formats are those the decode reads (sao.pub FlashMLA overview,
二、核心功能与架构: a 656-byte FP8 row is 512 FP8 NoPE values, 4 FP32 scales,
one per 128 values, and 64 BF16 RoPE values; 四、进阶玩法: the FP8 type is
float8_e4m3fn).  The pages say how a row is laid out, not how the scales
are chosen; the reading taken here is the usual absolute-max one:

  - per group g of 128 NoPE values: amax_g = max |x|, and
    scale_g = fp32(amax_g / 448), 448 being the largest e4m3fn magnitude;
  - code = the e4m3fn value nearest to fp32(x / scale_g), clamped to
    [-448, 448], ties to the even code (even mantissa), as in IEEE
    round-to-nearest-even;
  - amax_g = 0 gives scale_g = 0 and codes 0;
  - RoPE values are copied bit for bit; a BF16 pool row is the input row.

The two divisions are fp32 (the precision the kernel computes in); the
choice of the nearest code is then exact (fp64 comparisons against the
decoded table).  Input rows are bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np

ROW_BF16 = 1152
ROW_FP8 = 656


def _e4m3_table() -> np.ndarray:
    """Values of codes 0x00 .. 0x7E (the non-negative finite e4m3fn codes),
    from the format definition: exponent field E = bits 6..3 (bias 7),
    mantissa M = bits 2..0; E = 0 is subnormal, M * 2^-9."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = _e4m3_table()


def e4m3_code(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each finite v in [-448, 448], ties to the code
    with an even mantissa; the sign goes into bit 7 (-0.0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.searchsorted(_TABLE, a, side="left")          # first table value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _TABLE[lo]
    d_hi = _TABLE[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a == _TABLE[hi], hi, pick)
    sign = np.signbit(v).astype(np.int64) << 7
    return (pick.astype(np.int64) | sign).astype(np.uint8)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_row(row_bits: np.ndarray) -> np.ndarray:
    """One 576-value bf16 row (uint16 bits) -> its 656-byte FP8 row."""
    row_bits = np.asarray(row_bits, dtype=np.uint16)
    x = bf16_bits_to_f32(row_bits[:512]).reshape(4, 128)
    out = np.zeros(ROW_FP8, dtype=np.uint8)
    scales = np.zeros(4, dtype=np.float32)
    for g in range(4):
        amax = np.float32(np.max(np.abs(x[g])))
        scale = np.float32(amax / np.float32(448.0))
        scales[g] = scale
        if scale == 0:
            continue   # codes stay 0
        v = (x[g] / scale).astype(np.float32)
        v = np.clip(v, np.float32(-448.0), np.float32(448.0))
        out[128 * g:128 * (g + 1)] = e4m3_code(v)
    out[512:528] = scales.astype("<f4").view(np.uint8)
    out[528:656] = row_bits[512:576].astype("<u2").view(np.uint8)
    return out


def append(pool: np.ndarray, rows_bits: np.ndarray, slots: np.ndarray, fmt: int) -> np.ndarray:
    """The pool after writing token i to pool row slots[i] (page * 64 +
    position); negative or out-of-range slots write nothing.  pool is
    [num_pages * 64, row_bytes] uint8 and is not modified; a copy returns.
    fmt 0: bf16 rows (1152 bytes), fmt 1: 656-byte FP8 rows."""
    out = pool.copy()
    nrows = out.shape[0]
    rows_bits = np.asarray(rows_bits, dtype=np.uint16)
    for i, s in enumerate(np.asarray(slots).tolist()):
        if s < 0 or s >= nrows:
            continue
        if fmt == 0:
            out[s] = rows_bits[i].astype("<u2").view(np.uint8)
        else:
            out[s] = quantize_row(rows_bits[i])
    return out

"""The query as the FP8-MFMA variant of the decode uses it (TEST
INFRASTRUCTURE ONLY: the product library never calls it).

For FP8 pools the decode can run QK^T on the e4m3 MFMA with the query
quantised per row (sao.pub FlashMLA overview, 一、项目速览 and
二、核心功能与架构: the FP8 cache and its sparse-decode throughput).  The pages
do not say how the query is quantised; the reading taken here, per query
row and per half h of its 512 NoPE dims (dims 256 h .. 256 h + 255):

  - a power-of-two scale 2^p with p = e - 7, where 2^e <= amax < 2^(e+1)
    for amax = the half's largest |q| (p >= -126; p = 0 for an all-zero
    half), so every |q| / 2^p < 256;
  - codes c_d = the e4m3fn value nearest to q_d / 2^p, ties to the even
    code;
  - the quantised half q'_d = alpha * 2^p * c_d with the per-half factor
    alpha = (q . q) / (2^p c . q) (1 for an all-zero half), so that the
    rounding error q' - q is orthogonal to q: attention mostly weights keys
    along q, and this keeps the rounding from moving all their scores
    together;
  - the 64 RoPE dims are kept as they are.

The decode with the quantised query is then the plain definition (the
oracle's decode, fed the fp64 query) run on it.
"""
from __future__ import annotations

import numpy as np

from .kv_append import _TABLE, e4m3_code


def _values(q_bits):
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    return q.shape, (q.reshape(-1, 576).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def query_codes(q_bits: np.ndarray):
    """Per row and half: the e4m3 values times 2^p (before alpha), as fp64
    [..., 576] (RoPE dims kept), and the scales 2^p [..., 2]."""
    shape, vals = _values(q_bits)
    out = vals.copy()
    scales = np.ones((vals.shape[0], 2))
    for h in range(2):
        half = vals[:, 256 * h:256 * h + 256]
        amax = np.abs(half).max(axis=1)
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
        # exact exponent of amax (log2 of a bf16 value can round at a power of two)
        e = np.where(2.0 ** (e + 1) <= amax, e + 1, e)
        e = np.where(2.0 ** e > amax, e - 1, e)
        p = np.where(amax > 0, np.maximum(e - 7, -126), 0.0)
        s = 2.0 ** p
        codes = e4m3_code(half / s[:, None])
        mag = _TABLE[(codes & 0x7F).astype(np.int64)]
        sign = np.where(codes & 0x80, -1.0, 1.0)
        out[:, 256 * h:256 * h + 256] = sign * mag * s[:, None]
        scales[:, h] = s
    return out.reshape(shape), scales.reshape(shape[:-1] + (2,))


def quantize_query(q_bits: np.ndarray) -> np.ndarray:
    """q_bits: uint16 bf16 bits [..., 576]; returns the quantised query
    (fp64, same shape) with the per-half factor alpha applied."""
    shape, vals = _values(q_bits)
    qc, _ = query_codes(q_bits)
    qc = qc.reshape(-1, 576).copy()
    for h in range(2):
        sl = slice(256 * h, 256 * h + 256)
        qq = (vals[:, sl] * vals[:, sl]).sum(axis=1)
        qh = (qc[:, sl] * vals[:, sl]).sum(axis=1)
        alpha = np.where(qh > 0, qq / np.where(qh > 0, qh, 1.0), 1.0)
        qc[:, sl] *= alpha[:, None]
    return qc.reshape(shape)

"""fp64 CPU oracle for MLA paged-KV decoding.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never calls it and shares no code with it.

`decode` wraps the plain-C definition in mla_oracle.c (fp64, OpenMP over
query rows).  `schedule` is the split-KV schedule as a sequential walk.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import splitkv_schedule  # noqa: F401
from .splitkv_schedule import schedule, check_schedule, unit_blocks_dense, unit_blocks_sparse  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
# MLA_ORACLE_LIB selects another build of the same source (the sanitizer
# test loads an instrumented copy that way).
_LIB = os.environ.get("MLA_ORACLE_LIB") or os.path.join(_HERE, "libmla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FMA contraction so every
    product and sum rounds as written).  A build selected by MLA_ORACLE_LIB
    is the caller's and is left alone."""
    if os.environ.get("MLA_ORACLE_LIB"):
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_mla_decode.argtypes = [P, P, i, i, P, i, P, P, i, i, i, i,
                                          ctypes.c_float, i, i, P, P, P, i, P]
        lib.oracle_mla_decode.restype = i
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_decode_row.argtypes = [P, i, P]
        lib.oracle_decode_row.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def e4m3_to_double(code: int) -> float:
    return float(_load().oracle_e4m3_to_double(int(code)))


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def decode_row(row: np.ndarray, fmt: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    dst = np.empty(576, dtype=np.float64)
    _load().oracle_decode_row(_ptr(row), int(fmt), _ptr(dst))
    return dst


def decode_raw(q, kcache, fmt, block_table, seqlens, indices, softmax_scale,
               causal, sel=None, threads: int = 0, q_f64=None):
    """out [n, 512] fp64 and lse [n] fp64 for the selected flat query rows
    ((b*s_q + s)*h_q + h), or for all rows in order.  q_f64 (fp64, same
    shape as q) replaces the bf16 query values when given."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    if q_f64 is not None:
        q_f64 = np.ascontiguousarray(q_f64, dtype=np.float64)
        assert q_f64.shape == q.shape
    kcache = np.ascontiguousarray(kcache, dtype=np.uint8)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    batch, s_q, h_q, _ = q.shape
    topk = 0
    if indices is not None:
        indices = np.ascontiguousarray(indices, dtype=np.int32)
        topk = indices.shape[2]
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        n = sel.shape[0]
    else:
        n = batch * s_q * h_q
    out = np.empty((n, 512), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    st = lib.oracle_mla_decode(_ptr(q), _ptr(kcache), int(fmt), int(kcache.shape[0]),
                               _ptr(block_table), int(block_table.shape[1]), _ptr(seqlens),
                               _ptr(indices), int(topk), int(batch), int(s_q), int(h_q),
                               ctypes.c_float(softmax_scale), int(bool(causal)),
                               int(n if sel is not None else 0), _ptr(sel),
                               _ptr(out), _ptr(lse), int(threads), _ptr(q_f64))
    if st != 0:
        raise ValueError(f"oracle_mla_decode failed with status {st}")
    return out, lse


def decode(inp, sel=None, threads: int = 0, q_f64=None):
    """Run the oracle on an mla_inputs.Inputs bundle (with q_f64 in place
    of its query values when given)."""
    return decode_raw(inp.q, inp.kcache, inp.fmt, inp.block_table, inp.seqlens,
                      inp.indices, inp.softmax_scale, inp.causal, sel=sel,
                      threads=threads, q_f64=q_f64)


def merge_partials(lse_parts, o_parts):
    """Log-sum-exp merge of partial results over disjoint key sets (the
    pieces num_splits counts; topnet.top "Was ist FlashMLA?",
    "MLA-Metadaten abrufen"), in fp64.  lse_parts [k, n], o_parts
    [k, n, d], each piece's output normalised by its own row sum:
        lse = log sum_i exp(lse_i),  out = sum_i exp(lse_i - lse) * o_i,
    and out = 0, lse = -inf where every piece is empty (lse_i = -inf)."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(invalid="ignore"):
        w = np.exp(lse_parts - m_safe[None, :])          # exp(-inf) = 0
    total = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    weights = np.where(empty[None, :], 0.0, np.exp(lse_parts - np.where(empty, 0.0, lse)[None, :]))
    out = (weights[:, :, None] * o_parts).sum(axis=0)
    return out, lse

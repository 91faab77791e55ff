"""Python binding of libmla: argument marshalling only.

Every step of the decode runs in the HIP kernels behind the C ABI; torch
provides device memory and the current stream.  Names and call shapes follow
topnet.top "Was ist FlashMLA?", sections "MLA-Metadaten abrufen"
(get_mla_metadata(cache_seqlens, s_q * h_q // h_kv, h_kv)) and
"MLA-Decodierung ausfuehren" (decode with q, the KV cache, block_table,
cache_seqlens, dv, the metadata and a causal flag, returning out and lse).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _lib

D_QK = 576
D_V = 512
PAGE = 64


@dataclasses.dataclass
class MlaMetadata:
    """tile_scheduler_metadata and num_splits plus what produced them."""
    tile_metadata: torch.Tensor   # int32, device
    num_splits: torch.Tensor      # int32 [units + 1], device
    num_parts: int
    batch: int
    s_q: int
    q_rows_per_kv_head: int
    topk: int


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")


def get_mla_metadata(cache_seqlens: torch.Tensor, q_rows_per_kv_head: int, h_kv: int = 1,
                     s_q: int = 1, indices: Optional[torch.Tensor] = None,
                     num_parts: Optional[int] = None) -> MlaMetadata:
    """Split-KV schedule for one decode step, reused by every layer.

    q_rows_per_kv_head = s_q * h_q // h_kv.  For the sparse path pass
    `indices` ([batch, s_q, topk] int32) and s_q.  `num_parts` forces the
    number of parts (default: the library's choice for this device).
    """
    lib = _lib.load()
    _need_i32(cache_seqlens, "cache_seqlens")
    batch = cache_seqlens.shape[0]
    topk = 0
    if indices is not None:
        _need_i32(indices, "indices")
        if indices.dim() != 3 or indices.shape[0] != batch or indices.shape[1] != s_q:
            raise ValueError("indices must be [batch, s_q, topk]")
        topk = indices.shape[2]
    md_n = ctypes.c_size_t()
    ns_n = ctypes.c_size_t()
    if num_parts is None:
        P = ctypes.c_int()
        with torch.cuda.device(cache_seqlens.device):
            _lib.check(lib.mla_metadata_size(batch, s_q, q_rows_per_kv_head, h_kv, topk,
                                             ctypes.byref(P), ctypes.byref(md_n), ctypes.byref(ns_n)))
        num_parts = P.value
    else:
        _lib.check(lib.mla_metadata_size_for_parts(batch, s_q, topk, int(num_parts),
                                                   ctypes.byref(md_n), ctypes.byref(ns_n)))
    dev = cache_seqlens.device
    md = torch.empty(md_n.value, dtype=torch.int32, device=dev)
    ns = torch.empty(ns_n.value, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _lib.check(lib.mla_get_metadata(
            ctypes.c_void_p(cache_seqlens.data_ptr()),
            ctypes.c_void_p(indices.data_ptr() if indices is not None else None),
            batch, s_q, q_rows_per_kv_head, h_kv, topk, int(num_parts),
            ctypes.c_void_p(md.data_ptr()), ctypes.c_void_p(ns.data_ptr()),
            ctypes.c_void_p(_stream_ptr(dev))))
    return MlaMetadata(md, ns, int(num_parts), batch, s_q, q_rows_per_kv_head, topk)


def _kv_format(kcache: torch.Tensor) -> int:
    if kcache.dtype == torch.bfloat16 and kcache.shape[-1] == D_QK:
        return _lib.MLA_KV_BF16
    if kcache.dtype == torch.uint8 and kcache.shape[-1] == 656:
        return _lib.MLA_KV_FP8_656
    raise ValueError("kcache must be bf16 [pages, 64, 1, 576] or uint8 [pages, 64, 1, 656]")


def make_args(q, kcache, block_table, cache_seqlens, metadata: MlaMetadata, out, lse,
              softmax_scale=None, causal=False, indices=None, workspace=None,
              dv=D_V, qk_fp8=False) -> _lib.MlaDecodeArgs:
    if q.dim() != 4 or q.dtype != torch.bfloat16 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [batch, s_q, h_q, 576] tensor")
    if kcache.dim() != 4 or kcache.shape[1] != PAGE or not kcache.is_contiguous():
        raise ValueError("kcache must be a contiguous [num_pages, 64, h_kv, row] tensor")
    _need_i32(block_table, "block_table")
    _need_i32(cache_seqlens, "cache_seqlens")
    batch, s_q, h_q, d_qk = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be [batch, max_blocks]")
    if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] != batch:
        raise ValueError("cache_seqlens must be [batch]")
    if softmax_scale is None:
        softmax_scale = d_qk ** -0.5
    topk = 0
    if indices is not None:
        _need_i32(indices, "indices")
        if indices.dim() != 3 or tuple(indices.shape[:2]) != (batch, s_q):
            raise ValueError("indices must be [batch, s_q, topk]")
        topk = indices.shape[2]
    h_kv = kcache.shape[2]
    if (metadata.batch, metadata.s_q, metadata.topk) != (batch, s_q, topk) or \
            metadata.q_rows_per_kv_head != s_q * h_q // max(h_kv, 1):
        raise ValueError("metadata was built for other batch / s_q / heads / topk")
    if out.shape != (batch, s_q, h_q, int(dv)) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 [{batch}, {s_q}, {h_q}, {int(dv)}] tensor")
    if lse.shape != (batch, s_q, h_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous fp32 [{batch}, {s_q}, {h_q}] tensor")
    a = _lib.MlaDecodeArgs()
    a.batch, a.s_q, a.h_q, a.h_kv = batch, s_q, h_q, kcache.shape[2]
    a.d_qk, a.d_v, a.page_size = d_qk, int(dv), kcache.shape[1]
    a.num_pages, a.max_blocks_per_seq = kcache.shape[0], block_table.shape[1]
    a.topk = topk
    a.kv_format = _kv_format(kcache)
    a.softmax_scale = float(softmax_scale)
    a.causal = 1 if causal else 0
    a.num_parts = metadata.num_parts
    a.q = q.data_ptr()
    a.kcache = kcache.data_ptr()
    a.block_table = block_table.data_ptr()
    a.cache_seqlens = cache_seqlens.data_ptr()
    a.indices = indices.data_ptr() if indices is not None else None
    a.tile_metadata = metadata.tile_metadata.data_ptr()
    a.num_splits = metadata.num_splits.data_ptr()
    a.out = out.data_ptr()
    a.lse = lse.data_ptr()
    a.qk_fp8 = 1 if qk_fp8 else 0
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def workspace_bytes(args: _lib.MlaDecodeArgs) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().mla_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def mla_decode_kvcache(q: torch.Tensor, kcache: torch.Tensor, block_table: torch.Tensor,
                       cache_seqlens: torch.Tensor, softmax_scale: Optional[float] = None,
                       causal: bool = False, indices: Optional[torch.Tensor] = None,
                       metadata: Optional[MlaMetadata] = None, dv: int = D_V,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, qk_fp8: bool = False):
    """Decode one layer; returns (out [b, s_q, h_q, 512] bf16, lse [b, s_q, h_q] fp32).

    `metadata` is the step's schedule from get_mla_metadata, built once per
    decode step and passed to every layer; when it is omitted the schedule
    is built here on the same stream (one more kernel launch).  qk_fp8
    (FP8 pools, more than 32 query rows per unit): QK^T with the query
    quantised to e4m3 per row half (see mla_decode_args.qk_fp8)."""
    lib = _lib.load()
    batch, s_q, h_q, _ = q.shape
    dev = q.device
    if metadata is None:
        metadata = get_mla_metadata(cache_seqlens, s_q * h_q // max(kcache.shape[2], 1), kcache.shape[2],
                                    s_q=s_q, indices=indices)
    if out is None:
        out = torch.empty(batch, s_q, h_q, dv, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(batch, s_q, h_q, dtype=torch.float32, device=dev)
    args = make_args(q, kcache, block_table, cache_seqlens, metadata, out, lse,
                     softmax_scale=softmax_scale, causal=causal, indices=indices, dv=dv, qk_fp8=qk_fp8)
    with torch.cuda.device(dev):
        need = workspace_bytes(args)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
        _lib.check(lib.mla_decode_kvcache(ctypes.byref(args), ctypes.c_void_p(_stream_ptr(dev))))
    return out, lse


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(D_QK)


def refresh_mla_metadata(metadata: MlaMetadata, cache_seqlens: torch.Tensor,
                         indices: Optional[torch.Tensor] = None) -> MlaMetadata:
    """Rebuild the schedule into the existing metadata buffers (no
    allocation), e.g. at the start of every decode step."""
    lib = _lib.load()
    _need_i32(cache_seqlens, "cache_seqlens")
    if cache_seqlens.dim() != 1 or cache_seqlens.shape[0] != metadata.batch:
        raise ValueError("cache_seqlens batch differs from the metadata's")
    if (indices is None) != (metadata.topk == 0):
        raise ValueError("indices must be given exactly when the metadata is sparse")
    if indices is not None:
        _need_i32(indices, "indices")
        if tuple(indices.shape) != (metadata.batch, metadata.s_q, metadata.topk):
            raise ValueError("indices must be [batch, s_q, topk] as when the metadata was built")
    dev = cache_seqlens.device
    with torch.cuda.device(dev):
        _lib.check(lib.mla_get_metadata(
            ctypes.c_void_p(cache_seqlens.data_ptr()),
            ctypes.c_void_p(indices.data_ptr() if indices is not None else None),
            metadata.batch, metadata.s_q, metadata.q_rows_per_kv_head, 1, metadata.topk,
            metadata.num_parts, ctypes.c_void_p(metadata.tile_metadata.data_ptr()),
            ctypes.c_void_p(metadata.num_splits.data_ptr()), ctypes.c_void_p(_stream_ptr(dev))))
    return metadata


class DecodeCall:
    """A decode call with its arguments marshalled once: run() enqueues the
    whole decode, partial()/combine() its two kernels.  Holds references to
    every tensor it points at."""

    def __init__(self, q, kcache, block_table, cache_seqlens, metadata: MlaMetadata,
                 softmax_scale=None, causal=False, indices=None, out=None, lse=None,
                 workspace=None, qk_fp8=False):
        batch, s_q, h_q, _ = q.shape
        dev = q.device
        self.out = out if out is not None else torch.empty(batch, s_q, h_q, D_V, dtype=torch.bfloat16, device=dev)
        self.lse = lse if lse is not None else torch.empty(batch, s_q, h_q, dtype=torch.float32, device=dev)
        self.args = make_args(q, kcache, block_table, cache_seqlens, metadata, self.out, self.lse,
                              softmax_scale=softmax_scale, causal=causal, indices=indices, qk_fp8=qk_fp8)
        need = workspace_bytes(self.args)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.workspace = workspace
        self.args.workspace = workspace.data_ptr()
        self.args.workspace_bytes = workspace.numel() * workspace.element_size()
        self._keep = (q, kcache, block_table, cache_seqlens, metadata, indices)
        self.device = dev
        self._lib = _lib.load()

    def _call(self, fn):
        _lib.check(fn(ctypes.byref(self.args), ctypes.c_void_p(_stream_ptr(self.device))))

    def run(self):
        self._call(self._lib.mla_decode_kvcache)
        return self.out, self.lse

    def partial(self):
        self._call(self._lib.mla_decode_partial)

    def combine(self):
        self._call(self._lib.mla_decode_combine)

    def validate(self):
        """Synchronous debug audit of the device-resident inputs (block
        table pages, lengths, indices and the schedule); raises MlaError
        naming the first problem."""
        self._call(self._lib.mla_validate_inputs)


def validate_inputs(q, kcache, block_table, cache_seqlens, metadata: MlaMetadata,
                    causal=False, indices=None) -> None:
    """Debug check of a decode call's inputs before running it (synchronous;
    allocates the call's outputs and workspace).  Raises MlaError."""
    DecodeCall(q, kcache, block_table, cache_seqlens, metadata, causal=causal,
               indices=indices).validate()


def append_kv(rows: torch.Tensor, slots: torch.Tensor, kcache: torch.Tensor) -> torch.Tensor:
    """Write token i of rows ([n, 576] bf16) into pool row slots[i]
    (page * 64 + position; outside the pool: skipped) of kcache, as a bf16
    row or a quantised 656-byte FP8 row depending on kcache's format.
    Slots must be distinct (a repeated slot leaves its row unspecified).
    Returns kcache."""
    if rows.dim() != 2 or rows.shape[1] != D_QK or rows.dtype != torch.bfloat16 or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous bf16 [n, 576] tensor")
    _need_i32(slots, "slots")
    if slots.dim() != 1 or slots.shape[0] != rows.shape[0]:
        raise ValueError("slots must be [n] int32")
    if kcache.dim() != 4 or kcache.shape[1] != PAGE or not kcache.is_contiguous():
        raise ValueError("kcache must be a contiguous [num_pages, 64, 1, row] tensor")
    fmt = _kv_format(kcache)
    dev = rows.device
    with torch.cuda.device(dev):
        _lib.check(_lib.load().mla_append_kv(
            ctypes.c_void_p(rows.data_ptr()), ctypes.c_void_p(slots.data_ptr()), rows.shape[0], fmt,
            ctypes.c_void_p(kcache.data_ptr()), kcache.shape[0], ctypes.c_void_p(_stream_ptr(dev))))
    return kcache

"""Seeded synthetic inputs for MLA decoding over a 64-token paged KV cache.

This module only *constructs* inputs: sequence lengths, a shuffled page pool
with its block table, bf16 queries, the KV cache bytes (bf16 rows or the
656-byte FP8 rows), and top-k index lists.  It holds none of the decode's
arithmetic.  Both the fp64 oracle and the HIP library consume what it builds,
so the two sides always see byte-identical inputs.

Sources for the shapes and layouts:
  * topnet.top, "Was ist FlashMLA?", section "Hauptmerkmale": the KV cache is
    paged with a block size of 64 tokens, BF16 data.
  * topnet.top, same page, "MLA-Metadaten abrufen" / "MLA-Decodierung
    ausfuehren": cache_seqlens per sequence, a block_table, q of s_q tokens by
    h_q heads.
  * sao.pub FlashMLA overview, section "二、核心功能与架构": the FP8 cache row is
    512 FP8 NoPE values, 4 FP32 scale factors (one per 128 values) and 64
    unquantised BF16 RoPE values.
  * sao.pub, same section: a sparse `indices` tensor restricts the keys.

Quantiser reading (the pages name e4m3 but give no rounding rule): per group
of 128 NoPE values, scale = fp32(amax / 448), code = e4m3fn(RNE(clamp(x/scale,
+-448))); an all-zero group gets scale 0 and codes 0.  The decode only ever
reads the stored bytes, so these choices do not affect parity.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE = 64          # tokens per KV page
D_QK = 576         # 512 latent NoPE + 64 RoPE dims per query / key row
D_V = 512          # V is the first 512 dims of the shared latent row
D_NOPE = 512
D_ROPE = 64
FP8_ROW_BYTES = 656   # 512 e4m3 + 4 x fp32 scales + 64 x bf16
BF16_ROW_BYTES = 2 * D_QK

FMT_BF16 = 0
FMT_FP8 = 1

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F          # e4m3fn: exponent 15, mantissa 7
F32_NAN_BYTES = np.array([0x7FC00000], dtype="<u4").view(np.uint8)


@dataclasses.dataclass
class Config:
    """One workload.  `seqlens` is either a list, an int (all equal) or
    ("uniform", lo, hi) for an inclusive uniform draw."""
    name: str
    batch: int
    s_q: int
    h_q: int
    seqlens: object
    causal: bool = False
    fmt: int = FMT_BF16
    topk: int = 0
    masked_rows: int = 0       # sparse: how many batch rows get a -1 tail
    masked_tail: int = 0       # sparse: how many trailing entries become -1
    max_blocks: Optional[int] = None
    seed: int = 0
    topk_in_window: bool = False  # sparse + causal: draw each query's indices
                                  # from the keys it may see


# The five workloads the decode is measured and checked on, by short name.
# Seeds: 1000 for tiny, then 1001 .. 1006 in the order listed.
WORKLOADS = {
    "tiny": Config("tiny_b2_h16", batch=2, s_q=1, h_q=16, seqlens=[37, 130],
                   seed=1000),
    "membound": Config("membound_b64_h16_varlen", batch=64, s_q=1, h_q=16,
                       seqlens=("uniform", 1, 8192), max_blocks=128, seed=1001),
    "mtp": Config("mtp_b128_sq2_h128_causal", batch=128, s_q=2, h_q=128,
                  seqlens=4096, causal=True, seed=1002),
    "fp8": Config("fp8_b64_h128_L8192", batch=64, s_q=1, h_q=128, seqlens=8192,
                  fmt=FMT_FP8, seed=1003),
    "sparse": Config("sparse_fp8_b32_h128_L32768_top2048", batch=32, s_q=1, h_q=128,
                     seqlens=32768, fmt=FMT_FP8, topk=2048, masked_rows=8,
                     masked_tail=204, seed=1004),
    # Sparse prefill: 2048 new tokens at the end of an 8192-token sequence,
    # each attending to 2048 of the keys its causal window holds.
    "sparse_prefill": Config("sparse_prefill_fp8_b1_sq2048_h128_L8192_top2048", batch=1, s_q=2048,
                             h_q=128, seqlens=8192, causal=True, fmt=FMT_FP8, topk=2048,
                             topk_in_window=True, seed=1005),
    # Dense prefill: the same 2048 new tokens attending to their whole
    # causal window, bf16 rows.
    "dense_prefill": Config("dense_prefill_bf16_b1_sq2048_h128_L8192", batch=1, s_q=2048, h_q=128,
                            seqlens=8192, causal=True, seed=1006),
}


def row_bytes(fmt: int) -> int:
    return BF16_ROW_BYTES if fmt == FMT_BF16 else FP8_ROW_BYTES


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bits.
    Inputs are finite (they come from a normal draw)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_fp8_rows(nope: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """Pack tokens into 656-byte rows.

    nope: [n, 512] float32 source values; rope_bits: [n, 64] uint16 bf16 bits.
    Returns uint8 [n, 656] = 512 e4m3fn codes | 4 little-endian fp32 scales |
    64 little-endian bf16.  Uses torch's float8_e4m3fn cast (round to nearest
    even) for the code after clamping to the format's +-448 range.
    """
    import torch

    n = nope.shape[0]
    g = nope.reshape(n, 4, 128).astype(np.float32)
    amax = np.abs(g).max(axis=2)                           # [n, 4]
    scale = (amax / np.float32(448.0)).astype(np.float32)  # fp32(amax/448)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (g / safe[:, :, None]).astype(np.float32)
    y = np.clip(y, -448.0, 448.0).astype(np.float32)
    y = np.where(scale[:, :, None] > 0, y, np.float32(0.0)).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y.reshape(n, 512))).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    out = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:528] = np.ascontiguousarray(scale.astype("<f4")).view(np.uint8).reshape(n, 16)
    out[:, 528:656] = np.ascontiguousarray(rope_bits.astype("<u2")).view(np.uint8).reshape(n, 128)
    return out


@dataclasses.dataclass
class Inputs:
    cfg: Config
    q: np.ndarray              # uint16 bf16 bits [b, s_q, h_q, 576]
    kcache: np.ndarray         # uint8 [num_pages, 64, 1, row_bytes]
    block_table: np.ndarray    # int32 [b, max_blocks], -1 unused
    seqlens: np.ndarray        # int32 [b]
    indices: Optional[np.ndarray]  # int32 [b, s_q, topk] or None
    softmax_scale: float       # a value exactly representable in fp32
    causal: bool
    fmt: int

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def s_q(self):
        return self.q.shape[1]

    @property
    def h_q(self):
        return self.q.shape[2]

    @property
    def topk(self):
        return 0 if self.indices is None else self.indices.shape[2]

    @property
    def num_pages(self):
        return self.kcache.shape[0]

    def kv_bytes_read(self) -> int:
        """Algorithmic KV bytes: each visible key row once per sequence
        (dense), or once per listed valid index (sparse)."""
        rb = row_bytes(self.fmt)
        if self.indices is None:
            return int(self.seqlens.astype(np.int64).sum()) * rb
        tot = 0
        for b in range(self.batch):
            L = int(self.seqlens[b])
            idx = self.indices[b]
            tot += int(((idx >= 0) & (idx < L)).sum())
        return tot * rb

    def flops(self) -> int:
        """2*(576+512) FLOP per (query row, visible key)."""
        per = 2 * (D_QK + D_V)
        tot = 0
        for b in range(self.batch):
            L = int(self.seqlens[b])
            for s in range(self.s_q):
                W = min(max(L - self.s_q + 1 + s, 0), L) if self.causal else L
                if self.indices is None:
                    n = W
                else:
                    idx = self.indices[b, s]
                    n = int(((idx >= 0) & (idx < W)).sum())
                tot += n * self.h_q
        return tot * per


def _draw_seqlens(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    s = cfg.seqlens
    if isinstance(s, tuple) and s[0] == "uniform":
        return rng.integers(s[1], s[2] + 1, size=cfg.batch).astype(np.int32)
    if isinstance(s, int):
        return np.full(cfg.batch, s, dtype=np.int32)
    arr = np.asarray(s, dtype=np.int32)
    assert arr.shape == (cfg.batch,)
    return arr


def make_inputs(cfg: Config, seed: Optional[int] = None, poison: bool = False,
                extra_pages: int = 0, softmax_scale: Optional[float] = None,
                values: str = "normal") -> Inputs:
    """Build the inputs of one workload.

    Draw order: seqlens -> page permutation -> q -> kcache -> indices.
    poison=True fills every unused token slot (t >= L_b in a sequence's last
    page) and every extra guard page with NaN, so a decode that reads them
    shows it.  values="normal" draws N(0,1) in fp32 and rounds to bf16.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    seqlens = _draw_seqlens(cfg, rng)
    n_pages_b = [(int(L) + PAGE - 1) // PAGE for L in seqlens]
    used = int(sum(n_pages_b))
    num_pages = used + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    max_blocks = cfg.max_blocks or max(1, max(n_pages_b) if n_pages_b else 1)
    assert max_blocks >= max(n_pages_b + [0])
    block_table = np.full((cfg.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages_b):
        block_table[b, :n] = perm[off:off + n]
        off += n

    qf = rng.standard_normal((cfg.batch, cfg.s_q, cfg.h_q, D_QK), dtype=np.float32)
    q = f32_to_bf16_bits(qf)
    del qf

    rb = row_bytes(cfg.fmt)
    kcache = np.empty((num_pages, PAGE, 1, rb), dtype=np.uint8)
    # Fill page by page in chunks to bound peak host memory.
    chunk = 256
    for p0 in range(0, num_pages, chunk):
        p1 = min(num_pages, p0 + chunk)
        n_tok = (p1 - p0) * PAGE
        src = rng.standard_normal((n_tok, D_QK), dtype=np.float32)
        if cfg.fmt == FMT_BF16:
            kcache[p0:p1].reshape(n_tok, rb)[:] = f32_to_bf16_bits(src).view(np.uint8).reshape(n_tok, rb)
        else:
            rope = f32_to_bf16_bits(src[:, D_NOPE:])
            kcache[p0:p1].reshape(n_tok, rb)[:] = quantize_fp8_rows(src[:, :D_NOPE], rope)

    indices = None
    if cfg.topk > 0:
        indices = np.empty((cfg.batch, cfg.s_q, cfg.topk), dtype=np.int32)
        for b in range(cfg.batch):
            L = int(seqlens[b])
            for s in range(cfg.s_q):
                W = L
                if cfg.topk_in_window and cfg.causal:
                    W = min(max(L - cfg.s_q + 1 + s, 0), L)
                if W >= cfg.topk:
                    indices[b, s] = rng.choice(W, cfg.topk, replace=False).astype(np.int32)
                else:
                    row = np.full(cfg.topk, -1, dtype=np.int32)
                    row[:W] = rng.permutation(W).astype(np.int32)
                    indices[b, s] = row
        if cfg.masked_rows:
            rows = rng.choice(cfg.batch, cfg.masked_rows, replace=False)
            for b in rows:
                indices[b, :, cfg.topk - cfg.masked_tail:] = -1

    if poison:
        poison_cache(kcache, block_table, seqlens, cfg.fmt, used_pages=perm[:used])

    scale = float(np.float32(1.0 / math.sqrt(D_QK))) if softmax_scale is None else float(np.float32(softmax_scale))
    return Inputs(cfg=cfg, q=q, kcache=kcache, block_table=block_table,
                  seqlens=seqlens, indices=indices, softmax_scale=scale,
                  causal=cfg.causal, fmt=cfg.fmt)


def _nan_row(fmt: int) -> np.ndarray:
    if fmt == FMT_BF16:
        return np.full(D_QK, BF16_NAN, dtype="<u2").view(np.uint8)
    r = np.empty(FP8_ROW_BYTES, dtype=np.uint8)
    r[:512] = FP8_NAN
    r[512:528] = np.tile(F32_NAN_BYTES, 4)
    r[528:] = np.full(D_ROPE, BF16_NAN, dtype="<u2").view(np.uint8)
    return r


def poison_cache(kcache, block_table, seqlens, fmt, used_pages=None):
    """NaN every token slot no sequence owns: tails of last pages and pages
    that no block_table entry points to."""
    nan = _nan_row(fmt)
    owned = np.zeros(kcache.shape[0], dtype=bool)
    for b in range(block_table.shape[0]):
        L = int(seqlens[b])
        n = (L + PAGE - 1) // PAGE
        for j in range(n):
            owned[block_table[b, j]] = True
        if L % PAGE:
            kcache[block_table[b, n - 1], L % PAGE:, 0, :] = nan
    for p in np.nonzero(~owned)[0]:
        kcache[p, :, 0, :] = nan


def permute_pages(inp: Inputs, seed: int) -> Inputs:
    """Same logical cache with the physical pages shuffled and the block
    table rewritten to match."""
    rng = np.random.default_rng(seed)
    P = inp.num_pages
    perm = rng.permutation(P)            # new position of old page i is perm[i]
    newk = np.empty_like(inp.kcache)
    newk[perm] = inp.kcache
    bt = inp.block_table.copy()
    m = bt >= 0
    bt[m] = perm[bt[m]]
    return dataclasses.replace(inp, kcache=newk, block_table=bt)


def small_config(batch, s_q, h_q, seqlens, causal=False, fmt=FMT_BF16, topk=0,
                 seed=7, max_blocks=None, topk_in_window=False):
    return Config(name="custom", batch=batch, s_q=s_q, h_q=h_q,
                  seqlens=list(seqlens), causal=causal, fmt=fmt, topk=topk,
                  seed=seed, max_blocks=max_blocks, topk_in_window=topk_in_window)

"""Invariants of the GPU result itself (no oracle in the comparison): the
order of sparse indices does not matter, masked (-1) entries are the same
as absent ones, and a shared RoPE row with a zero NoPE query gives the
closed form out = mean of the visible V rows, lse = c + ln N."""
import dataclasses

import numpy as np
import pytest

import mla_inputs as gen
from gpu_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_sparse_index_order_does_not_matter(fmt):
    cfg = gen.small_config(3, 2, 16, [500, 90, 1200], causal=True, fmt=fmt, topk=150, seed=71)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    rng = np.random.default_rng(71)
    shuffled = inp.indices.copy()
    for b in range(3):
        for s in range(2):
            shuffled[b, s] = rng.permutation(shuffled[b, s])
    log(f"index order fmt={fmt}")
    o1, l1, _ = run_gpu(inp, num_parts=8)
    o2, l2, _ = run_gpu(dataclasses.replace(inp, indices=shuffled), num_parts=8)
    compare(o2, l2, o1, l1, fmt, "shuffled indices")


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_masked_entries_equal_removed_ones(fmt):
    cfg = gen.small_config(2, 1, 128, [700, 300], fmt=fmt, topk=100, seed=72)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    rng = np.random.default_rng(72)
    # the same 100 entries with 60 masked ones (-1 and out of range) mixed in
    padded = np.empty((2, 1, 160), dtype=np.int32)
    for b, L in enumerate([700, 300]):
        junk = np.concatenate([np.full(30, -1), rng.integers(L, L + 500, 30)]).astype(np.int32)
        row = np.concatenate([inp.indices[b, 0], junk])
        padded[b, 0] = row[rng.permutation(160)]
    log(f"masked entries fmt={fmt}")
    o1, l1, _ = run_gpu(inp, num_parts=16)
    o2, l2, _ = run_gpu(dataclasses.replace(inp, indices=padded, cfg=dataclasses.replace(inp.cfg, topk=160)),
                        num_parts=16)
    compare(o2, l2, o1, l1, fmt, "masked entries")


def _shared_rope_inputs(h_q, s_q, seqlens, causal, seed):
    """bf16 pool whose rows share one RoPE vector (dims 512..575) and have
    random NoPE; q is zero on NoPE and random on RoPE, so every visible key
    scores c = scale * q_rope . k_rope."""
    cfg = gen.small_config(len(seqlens), s_q, h_q, seqlens, causal=causal, seed=seed)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=1)
    rng = np.random.default_rng(seed)
    rope = gen.f32_to_bf16_bits(rng.standard_normal(64).astype(np.float32))
    kv = inp.kcache.view(np.uint16).reshape(inp.num_pages, 64, 576)
    kv[:, :, 512:] = rope
    q = inp.q.reshape(-1, 576)
    q[:, :512] = 0
    return inp, rope


@pytest.mark.parametrize("h_q,s_q,causal", [(16, 1, False), (128, 2, True)])
def test_shared_rope_gives_mean_of_v(h_q, s_q, causal):
    seqlens = [1, 64, 333, 1000]
    inp, rope = _shared_rope_inputs(h_q, s_q, seqlens, causal, 73)
    log(f"shared rope h_q={h_q} s_q={s_q} causal={causal}")
    o, l, _ = run_gpu(inp, num_parts=8)
    o = o.reshape(len(seqlens), s_q, h_q, 512)
    l = l.reshape(len(seqlens), s_q, h_q)
    kr = gen.bf16_bits_to_f32(rope).astype(np.float64)
    kv = inp.kcache.view(np.uint16).reshape(inp.num_pages, 64, 576)
    q = inp.q.reshape(len(seqlens), s_q, h_q, 576)
    for b, L in enumerate(seqlens):
        rows = np.stack([kv[inp.block_table[b, t // 64], t % 64, :512] for t in range(L)])
        v = gen.bf16_bits_to_f32(rows).astype(np.float64)
        for s in range(s_q):
            W = min(max(L - s_q + 1 + s, 0), L) if causal else L
            if W == 0:   # no visible key: out 0, lse -inf
                assert np.all(np.isneginf(l[b, s])) and not o[b, s].any()
                continue
            mean = v[:W].mean(axis=0)
            # split sequences merge bf16 partial means, each within 2^-9 of
            # its value, and |partial mean| <= max |v| over the visible keys
            vmax = np.abs(v[:W]).max(axis=0)
            for h in range(h_q):
                qr = gen.bf16_bits_to_f32(q[b, s, h, 512:]).astype(np.float64)
                c = float(np.float32(inp.softmax_scale)) * float(qr @ kr)
                # every score is the same fp32 value, so every probability
                # rounds to 1: out is the mean of V up to bf16 rounding of
                # the result and of split partials, and lse = c + ln W
                assert abs(l[b, s, h] - (c + np.log(W))) <= 1e-4 * max(1.0, abs(c)), (b, s, h)
                bound = 2 ** -8 * np.abs(mean) + 2 ** -8 * vmax + 1e-6
                assert np.all(np.abs(o[b, s, h] - mean) <= bound), (b, s, h)

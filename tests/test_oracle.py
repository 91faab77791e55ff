"""Pins for the fp64 oracle (CPU only).

The pages print no worked example, so the oracle is pinned to things outside
itself:
  * brute force: the paged cache is unrolled by walking block_table in torch,
    rows are decoded with torch's bfloat16 / float8_e4m3fn types, and the
    attention is torch's scaled_dot_product_attention in fp64 (the one-KV-head
    case is ordinary attention with v = k[..., :512]); lse from
    torch.logsumexp;
  * closed forms: q = 0 gives lse = ln N and out = mean(V); a single key
    returns its V row exactly; equal scores give the mean of V;
  * invariants: page permutation, NoPE/RoPE separation, sparse with every
    index equals dense, -1 entries are removals, repeated indices count twice.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_inputs as gen


def torch_rows(inp, b):
    """Unpaged fp64 key rows [L_b, 576] of sequence b, decoded by torch."""
    L = int(inp.seqlens[b])
    n = (L + 63) // 64
    pages = inp.block_table[b, :n]
    rb = gen.row_bytes(inp.fmt)
    raw = inp.kcache[pages].reshape(n * 64, rb)[:L]
    if inp.fmt == gen.FMT_BF16:
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64)
    codes = torch.from_numpy(np.ascontiguousarray(raw[:, :512])).view(torch.float8_e4m3fn).to(torch.float64)
    scales = torch.from_numpy(np.ascontiguousarray(raw[:, 512:528]).view("<f4").astype(np.float64))
    rope = torch.from_numpy(np.ascontiguousarray(raw[:, 528:]).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    nope = codes * scales.repeat_interleave(128, dim=1)
    return torch.cat([nope, rope], dim=1)


def brute(inp):
    """Reference by library routines; returns out [rows,512], lse [rows]."""
    B, S, H = inp.batch, inp.s_q, inp.h_q
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    out = torch.zeros(B, S, H, 512, dtype=torch.float64)
    lse = torch.full((B, S, H), -math.inf, dtype=torch.float64)
    for b in range(B):
        K = torch_rows(inp, b)
        L = int(inp.seqlens[b])
        for s in range(S):
            W = min(max(L - S + 1 + s, 0), L) if inp.causal else L
            if inp.indices is None:
                keys = list(range(W))
            else:
                keys = [int(t) for t in inp.indices[b, s] if 0 <= int(t) < W]
            if not keys:
                continue
            Ks = K[keys]
            qs = q[b, s]
            o = torch.nn.functional.scaled_dot_product_attention(
                qs[None, None], Ks[None, None], Ks[None, None, :, :512], scale=inp.softmax_scale)
            out[b, s] = o[0, 0]
            lse[b, s] = torch.logsumexp(inp.softmax_scale * (qs @ Ks.T), dim=-1)
    return out.reshape(-1, 512).numpy(), lse.reshape(-1).numpy()


def assert_close_to_brute(oracle_mod, inp, rtol=1e-10, atol=1e-12):
    o, l = oracle_mod.decode(inp, threads=4)
    bo, bl = brute(inp)
    assert np.array_equal(np.isinf(l), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(l[fin], bl[fin], rtol=rtol, atol=atol)
    np.testing.assert_allclose(o, bo, rtol=rtol, atol=atol)
    return o, l


def test_tiny_workload_matches_brute_force(oracle_mod):
    inp = gen.make_inputs(gen.WORKLOADS["tiny"], poison=True)
    assert list(inp.seqlens) == [37, 130] and inp.num_pages == 4
    assert sorted(inp.block_table[inp.block_table >= 0].tolist()) == [0, 1, 2, 3]
    assert_close_to_brute(oracle_mod, inp)


def _random_cases(n=40):
    rng = np.random.default_rng(12345)
    cases = []
    for i in range(n):
        b = int(rng.integers(1, 4))
        s_q = int(rng.integers(1, 4))
        h_q = int(rng.choice([1, 3, 16]))
        seqlens = [int(x) for x in rng.integers(0, 301, size=b)]
        causal = bool(rng.integers(0, 2))
        fmt = int(rng.integers(0, 2))
        topk = int(rng.choice([0, 0, 7, 64, 100]))
        cases.append((b, s_q, h_q, seqlens, causal, fmt, topk, 100 + i))
    return cases


@pytest.mark.parametrize("case", _random_cases())
def test_random_small_shapes_match_brute_force(oracle_mod, case):
    b, s_q, h_q, seqlens, causal, fmt, topk, seed = case
    cfg = gen.small_config(b, s_q, h_q, seqlens, causal=causal, fmt=fmt, topk=topk, seed=seed)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    if topk:
        # mix in out-of-range and negative entries, which must be masked
        rng = np.random.default_rng(seed)
        mask = rng.random(inp.indices.shape) < 0.2
        inp.indices[mask] = rng.integers(-5, 400, size=int(mask.sum()))
    assert_close_to_brute(oracle_mod, inp)


def test_page_permutation_is_bitwise_invariant(oracle_mod):
    for fmt in (gen.FMT_BF16, gen.FMT_FP8):
        cfg = gen.small_config(3, 2, 4, [5, 130, 257], causal=True, fmt=fmt, seed=3)
        inp = gen.make_inputs(cfg, poison=True, extra_pages=3)
        o1, l1 = oracle_mod.decode(inp)
        o2, l2 = oracle_mod.decode(gen.permute_pages(inp, 99))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_single_key_returns_its_v_row_exactly(oracle_mod):
    cfg = gen.small_config(2, 1, 16, [1, 1], seed=4)
    inp = gen.make_inputs(cfg, poison=True)
    o, l = oracle_mod.decode(inp)
    for b in range(2):
        page = inp.block_table[b, 0]
        v = gen.bf16_bits_to_f32(inp.kcache[page, 0, 0].view(np.uint16)).astype(np.float64)
        qb = gen.bf16_bits_to_f32(inp.q[b, 0]).astype(np.float64)
        for h in range(16):
            assert np.array_equal(o[b * 16 + h], v[:512])
            ref = inp.softmax_scale * float(np.dot(qb[h], v))
            assert abs(l[b * 16 + h] - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_zero_query_counts_visible_keys(oracle_mod, fmt):
    """q = 0: every score is 0, so lse = ln(#visible keys) and out is the
    plain mean of the visible V rows.  Causal s_q=2 sees L-1 then L keys."""
    seqlens = [1, 63, 64, 65, 127, 128, 129, 200]
    cfg = gen.small_config(len(seqlens), 2, 2, seqlens, causal=True, fmt=fmt, seed=5)
    inp = gen.make_inputs(cfg, poison=True)
    inp.q[:] = 0
    o, l = oracle_mod.decode(inp)
    o = o.reshape(len(seqlens), 2, 2, 512)
    l = l.reshape(len(seqlens), 2, 2)
    for b, L in enumerate(seqlens):
        K = torch_rows(inp, b).numpy()
        for s in range(2):
            n = L - 1 + s
            if n == 0:
                assert np.all(l[b, s] == -np.inf) and np.all(o[b, s] == 0)
                continue
            assert np.allclose(l[b, s], math.log(n), rtol=0, atol=1e-14)
            np.testing.assert_allclose(o[b, s, 0], K[:n, :512].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_equal_scores_give_mean_of_v(oracle_mod):
    """RoPE-only scores: q is zero on the 512 NoPE dims and every key shares
    one RoPE vector, so all scores equal c = sigma * q_rope . k_rope."""
    cfg = gen.small_config(1, 1, 3, [150], seed=6)
    inp = gen.make_inputs(cfg, poison=True)
    inp.q[..., :512] = 0
    page_rows = inp.kcache.view(np.uint16).reshape(inp.num_pages, 64, 576)
    shared = page_rows[inp.block_table[0, 0], 0, 512:].copy()
    for j in range(3):
        page_rows[inp.block_table[0, j], :, 512:] = shared
    o, l = oracle_mod.decode(inp)
    K = torch_rows(inp, 0).numpy()
    qb = gen.bf16_bits_to_f32(inp.q[0, 0]).astype(np.float64)
    for h in range(3):
        c = inp.softmax_scale * float(np.dot(qb[h, 512:], K[0, 512:]))
        assert abs(l[h] - (c + math.log(150))) <= 1e-12
        np.testing.assert_allclose(o[h], K[:, :512].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_rope_dims_enter_the_score(oracle_mod):
    """With q zero on the RoPE dims, zeroing every key's RoPE part changes
    nothing; with q non-zero there it does."""
    cfg = gen.small_config(2, 1, 4, [70, 140], seed=8)
    inp = gen.make_inputs(cfg)
    base = dataclasses.replace(inp, q=inp.q.copy(), kcache=inp.kcache.copy())
    base.q[..., 512:] = 0
    o1, l1 = oracle_mod.decode(base)
    z = dataclasses.replace(base, kcache=base.kcache.copy())
    z.kcache.view(np.uint16).reshape(-1, 576)[:, 512:] = 0
    o2, l2 = oracle_mod.decode(z)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle_mod.decode(inp)
    z2 = dataclasses.replace(inp, kcache=z.kcache)
    o4, l4 = oracle_mod.decode(z2)
    assert not np.allclose(l3, l4)


def test_sparse_all_indices_equals_dense(oracle_mod):
    for fmt in (gen.FMT_BF16, gen.FMT_FP8):
        seqlens = [100, 64, 37]
        cfg = gen.small_config(3, 2, 4, seqlens, causal=True, fmt=fmt, seed=9)
        dense = gen.make_inputs(cfg, poison=True)
        idx = np.full((3, 2, 120), -1, dtype=np.int32)
        for b, L in enumerate(seqlens):
            idx[b, :, :L] = np.arange(L)
        sp = dataclasses.replace(dense, indices=idx)
        od, ld = oracle_mod.decode(dense)
        os_, ls = oracle_mod.decode(sp)
        assert np.array_equal(od, os_) and np.array_equal(ld, ls)
        # shuffled order: equal up to rounding order
        rng = np.random.default_rng(1)
        idx2 = idx.copy()
        for b in range(3):
            for s in range(2):
                rng.shuffle(idx2[b, s])
        o2, l2 = oracle_mod.decode(dataclasses.replace(dense, indices=idx2))
        np.testing.assert_allclose(o2, od, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l2, ld, rtol=1e-13, atol=1e-14)


def test_sparse_duplicate_index_counts_twice(oracle_mod):
    cfg = gen.small_config(1, 1, 2, [90], fmt=gen.FMT_FP8, topk=11, seed=10)
    inp = gen.make_inputs(cfg)
    inp.q[:] = 0
    idx = inp.indices
    idx[0, 0, 10] = idx[0, 0, 3]   # entry 3 now listed twice among 11
    o, l = oracle_mod.decode(inp)
    K = torch_rows(inp, 0).numpy()
    keys = [int(t) for t in idx[0, 0]]
    assert abs(l[0] - math.log(11)) < 1e-14
    np.testing.assert_allclose(o[0], K[keys, :512].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_empty_key_sets(oracle_mod):
    cfg = gen.small_config(3, 2, 2, [0, 1, 5], causal=True, topk=0, seed=11)
    inp = gen.make_inputs(cfg)
    o, l = oracle_mod.decode(inp)
    l = l.reshape(3, 2, 2)
    assert np.all(l[0] == -np.inf)            # L = 0
    assert np.all(l[1, 0] == -np.inf)         # causal window 0
    assert np.all(np.isfinite(l[1, 1])) and np.all(np.isfinite(l[2]))
    assert np.all(o.reshape(3, 2, 2, 512)[0] == 0)
    sp = gen.make_inputs(gen.small_config(1, 1, 2, [50], topk=8, seed=12))
    sp.indices[:] = -1
    o, l = oracle_mod.decode(sp)
    assert np.all(l == -np.inf) and np.all(o == 0)


def test_selected_rows_match_full_run(oracle_mod):
    cfg = gen.small_config(2, 2, 3, [77, 200], causal=True, seed=13)
    inp = gen.make_inputs(cfg, poison=True)
    o, l = oracle_mod.decode(inp)
    sel = np.array([11, 0, 5, 7], dtype=np.int32)
    os_, ls = oracle_mod.decode(inp, sel=sel)
    assert np.array_equal(os_, o[sel]) and np.array_equal(ls, l[sel])


def test_bad_block_table_is_reported(oracle_mod):
    cfg = gen.small_config(1, 1, 1, [70], seed=14)
    inp = gen.make_inputs(cfg)
    inp.block_table[0, 1] = inp.num_pages + 5
    with pytest.raises(ValueError):
        oracle_mod.decode(inp)


def test_merge_of_disjoint_key_sets_equals_the_whole(oracle_mod):
    """Log-sum-exp merge identity, pinned on the decode oracle itself: split
    every sequence's keys into three disjoint sets (sparse index lists),
    decode each set alone and merge the pieces; the result equals the dense
    decode over all keys.  Empty pieces (lse = -inf) drop out; a row whose
    pieces are all empty merges to out = 0, lse = -inf."""
    seqlens = [130, 1, 77, 0]
    cfg = gen.small_config(len(seqlens), 1, 4, seqlens, seed=21)
    inp = gen.make_inputs(cfg)
    o_all, l_all = oracle_mod.decode(inp)
    rng = np.random.default_rng(4)
    topk = max(seqlens)
    pieces_o, pieces_l = [], []
    owner = [rng.integers(0, 3, size=L) for L in seqlens]   # piece of every key
    for piece in range(3):
        idx = np.full((len(seqlens), 1, topk), -1, dtype=np.int32)
        for b, L in enumerate(seqlens):
            keys = np.nonzero(owner[b] == piece)[0]
            idx[b, 0, :keys.size] = keys
        o, l = oracle_mod.decode(dataclasses.replace(inp, indices=idx))
        pieces_o.append(o)
        pieces_l.append(l)
    out, lse = oracle_mod.merge_partials(np.stack(pieces_l), np.stack(pieces_o))
    fin = np.isfinite(l_all)
    assert np.array_equal(np.isneginf(lse), np.isneginf(l_all))
    np.testing.assert_allclose(lse[fin], l_all[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, o_all, rtol=1e-11, atol=1e-13)
    assert np.all(out[~fin] == 0)


def test_merge_closed_forms(oracle_mod):
    """Two pieces of equal lse c: lse = c + ln 2, out = the mean of the two;
    one piece: itself; a piece of lse -inf: no weight."""
    o = np.array([[[1.0, -2.0]], [[3.0, 4.0]]])
    out, lse = oracle_mod.merge_partials(np.array([[0.5], [0.5]]), o)
    assert abs(lse[0] - (0.5 + math.log(2))) <= 1e-15
    np.testing.assert_allclose(out[0], [2.0, 1.0], rtol=0, atol=1e-15)
    out, lse = oracle_mod.merge_partials(np.array([[-1.25], [-np.inf]]), o)
    assert lse[0] == -1.25 and np.array_equal(out[0], [1.0, -2.0])
    out, lse = oracle_mod.merge_partials(np.array([[-np.inf], [-np.inf]]), o)
    assert np.isneginf(lse[0]) and np.all(out[0] == 0)

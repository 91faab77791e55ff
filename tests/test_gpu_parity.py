"""GPU parity of the HIP decode path against the fp64 oracle.

Everything here goes through the Python binding into libmla's C ABI.
Tolerances are in gpu_util.TOL.
"""
import dataclasses

import numpy as np
import pytest

import mla_inputs as gen
from gpu_util import compare, log, run_gpu, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_metadata_amd as m
    m.load_library()


def test_tiny_workload(oracle_mod):
    inp = gen.make_inputs(gen.WORKLOADS["tiny"], poison=True)
    o, l, md = run_gpu(inp)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, inp.fmt, "tiny", inp=inp)


def _cases():
    rng = np.random.default_rng(2024)
    out = []
    for i in range(48):
        b = int(rng.integers(1, 5))
        s_q = int(rng.choice([1, 1, 2, 3]))
        h_q = int(rng.choice([1, 5, 16, 16, 20, 64, 128]))
        seqlens = [int(x) for x in rng.integers(0, 301, size=b)]
        causal = bool(rng.integers(0, 2))
        fmt = int(rng.integers(0, 2))
        topk = int(rng.choice([0, 0, 0, 7, 64, 100, 130]))
        parts = [None, 1, 8, 24][i % 4]
        out.append((b, s_q, h_q, seqlens, causal, fmt, topk, parts, 500 + i))
    return out


@pytest.mark.parametrize("case", _cases())
def test_random_small_shapes(oracle_mod, case):
    b, s_q, h_q, seqlens, causal, fmt, topk, parts, seed = case
    cfg = gen.small_config(b, s_q, h_q, seqlens, causal=causal, fmt=fmt, topk=topk, seed=seed)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    if topk:
        rng = np.random.default_rng(seed)
        mask = rng.random(inp.indices.shape) < 0.2
        inp.indices[mask] = rng.integers(-5, 400, size=int(mask.sum()))
    log(f"case b={b} s_q={s_q} h_q={h_q} L={seqlens} causal={causal} fmt={fmt} topk={topk} parts={parts}")
    o, l, _ = run_gpu(inp, num_parts=parts)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, fmt, "random", inp=inp)


# h_q 16: 16-row tiles (dense R = 32); 17: dense R = 34, the smallest 128-row
# tile case, sparse R = 17, a second 16-row tile of one row; 64: 128-row tiles
@pytest.mark.parametrize("h_q", [16, 17, 64])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("topk", [0, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_combination_matrix(oracle_mod, h_q, fmt, topk, causal):
    """Every pairing of tile width, KV format, dense or sparse keys and
    causal masking at least once, with two query tokens, lengths 0, 1, a
    page and a bit, and a few pages, forced splits and poisoned unused slots."""
    seed = 3000 + 8 * (h_q == 64) + 16 * (h_q == 17) + 4 * fmt + 2 * (topk > 0) + int(causal)
    cfg = gen.small_config(4, 2, h_q, [0, 1, 65, 300], causal=causal, fmt=fmt, topk=topk, seed=seed)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    if topk:
        rng = np.random.default_rng(seed)
        mask = rng.random(inp.indices.shape) < 0.2
        inp.indices[mask] = rng.integers(-5, 400, size=int(mask.sum()))
    log(f"matrix h_q={h_q} fmt={fmt} topk={topk} causal={causal}")
    o, l, md = run_gpu(inp, num_parts=8)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, fmt, f"matrix h_q={h_q} fmt={fmt} topk={topk} causal={causal}", inp=inp)


@pytest.mark.parametrize("parts", [1, 7, 8, 256, 1024])
def test_num_parts_sweep(oracle_mod, parts):
    cfg = gen.small_config(3, 2, 16, [700, 64, 1300], causal=True, seed=31)
    inp = gen.make_inputs(cfg, poison=True)
    o, l, _ = run_gpu(inp, num_parts=parts)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, inp.fmt, f"parts={parts}", inp=inp)


def test_schedule_matches_oracle_bitwise():
    from oracle import splitkv_schedule as S
    rng = np.random.default_rng(77)
    for trial in range(16):
        # trials 12..15: more than 1024 units (several scan chunks), the
        # largest part count, and index rows that are not 16-byte multiples
        b = int(rng.integers(1, 300)) if trial < 12 else int(rng.integers(1025, 2600))
        sl = rng.integers(0, 20000, size=b).astype(np.int32)
        P = int(rng.choice([1, 8, 13, 256, 1000])) if trial < 12 else int(rng.choice([7, 2048]))
        sparse = trial % 3 == 2
        s_q = 2 if sparse else 1
        import torch as T
        slt = T.from_numpy(sl).cuda()
        idx = None
        if sparse:
            topk = 300 if trial < 12 else 61
            ind = rng.integers(-2, 25000, size=(b, s_q, topk)).astype(np.int32)
            idx = T.from_numpy(ind).cuda()
            nb = S.unit_blocks_sparse(sl, ind)
        else:
            nb = S.unit_blocks_dense(sl)
        from mla_paged_kv_metadata_amd import get_mla_metadata
        md = get_mla_metadata(slt, s_q * 16, 1, s_q=s_q, indices=idx, num_parts=P)
        T.cuda.synchronize()
        ref_md, ref_ns = S.schedule(nb, P, 2, unit_len=np.repeat(sl, s_q) if sparse else sl)
        assert np.array_equal(md.tile_metadata.cpu().numpy(), ref_md), trial
        assert np.array_equal(md.num_splits.cpu().numpy(), ref_ns), trial
        S.check_schedule(ref_md, ref_ns, nb)


@pytest.mark.parametrize("units,sparse", [(1, True), (63, True), (64, True), (65, True), (4096, True),
                                          (4097, True), (65, False), (4096, False), (4097, False),
                                          (6000, False), (70000, True)])
def test_schedule_unit_count_boundaries(units, sparse):
    """Unit counts on both sides of the schedule kernel's switches: at most
    64 sparse units read in one pass, and the first 4096 units' counts and
    lengths kept on chip (the rest read back from memory).  Sparse rows get
    masked tails of random length so that some need the longer scan."""
    from oracle import splitkv_schedule as S
    import torch as T
    from mla_paged_kv_metadata_amd import get_mla_metadata
    rng = np.random.default_rng(1000 + units + sparse)
    s_q = 1
    if sparse:
        s_q = 3 if units % 3 == 0 else 1
        if units > 65536:   # past the done bits of the one-entry pass: one sequence, many query tokens
            s_q = units
    b = units // s_q
    sl = rng.integers(0, 9000, size=b).astype(np.int32)
    idx = None
    if sparse:
        topk = 520 if units <= 65 else (132 if units <= 65536 else 72)
        ind = rng.integers(0, 9000, size=(b, s_q, topk)).astype(np.int32) % np.maximum(sl, 1)[:, None, None]
        cut = rng.integers(0, topk + 1, size=(b, s_q))
        for i in range(b):
            for s in range(s_q):
                if rng.random() < 0.5:
                    ind[i, s, cut[i, s]:] = -1
        idx = T.from_numpy(ind).cuda()
        nb = S.unit_blocks_sparse(sl, ind)
    else:
        nb = S.unit_blocks_dense(sl)
    log(f"schedule boundary units={units} sparse={sparse}")
    for P in (8, 256, 2048):
        md = get_mla_metadata(T.from_numpy(sl).cuda(), s_q * 16, 1, s_q=s_q, indices=idx, num_parts=P)
        T.cuda.synchronize()
        ref_md, ref_ns = S.schedule(nb, P, 2, unit_len=np.repeat(sl, s_q) if sparse else sl)
        assert np.array_equal(md.tile_metadata.cpu().numpy(), ref_md), P
        assert np.array_equal(md.num_splits.cpu().numpy(), ref_ns), P


def _schedule_by_positions(nb, P, c0, unit_len):
    """The schedule's rows and split counts from its definition (block j of
    unit u sits at position C_u + c0 + j and belongs to part pos // T),
    evaluated per part at its two boundary positions in int64 instead of
    walking every block, so that it reaches cost lines past 2^31."""
    nb = np.asarray(nb, dtype=np.int64)
    C = np.concatenate([[0], np.cumsum(nb + c0)[:-1]])
    total = int(nb.sum()) + c0 * len(nb)
    T = max(1, -(-total // P)) if total > 0 else 1
    first = C + c0
    f, l = first // T, (first + nb - 1) // T
    ns = np.concatenate([[0], np.cumsum(l - f + 1)]).astype(np.int32)
    md = np.zeros(8 + 8 * P + len(nb), dtype=np.int64)
    md[:8] = [P, T, c0, len(nb), int(nb.sum()), 0x4D4C4131, 0, 0]
    md[8 + 8 * P:] = nb
    for p in range(P):
        us = np.nonzero((f <= p) & (l >= p))[0]
        row = [-1, 0, -1, 0, 0, 0, 0, 0]
        if us.size:
            u0, u1 = int(us[0]), int(us[-1])
            row = [u0, max(0, p * T - int(first[u0])), u1, min(int(nb[u1]), (p + 1) * T - int(first[u1])),
                   p - int(f[u0]), int(unit_len[u0]), int(nb[u0]), 0]
        md[8 + 8 * p: 16 + 8 * p] = row
    return md.astype(np.int32), ns


def test_schedule_by_positions_matches_the_walk():
    """Pins the boundary-position evaluation above to the oracle's walk."""
    from oracle import splitkv_schedule as S
    rng = np.random.default_rng(4242)
    for trial in range(40):
        U = int(rng.integers(1, 60))
        nb = rng.integers(1, 300, size=U) if trial % 2 else rng.integers(1, 4, size=U)
        P = int(rng.choice([1, 3, 8, 64, 255, 2048]))
        ul = rng.integers(0, 20000, size=U)
        want_md, want_ns = S.schedule(nb, P, 2, unit_len=ul)
        got_md, got_ns = _schedule_by_positions(nb, P, 2, ul)
        assert np.array_equal(got_md, want_md) and np.array_equal(got_ns, want_ns), trial


@pytest.mark.parametrize("units,last_blocks", [(65, 61), (65, 62), (4000, None)])
def test_schedule_cost_line_at_2_31(units, last_blocks):
    """Cost lines that end at 2^31 - 1, exactly 2^31, and past it (4000
    units in four scan chunks, fewer than 2^31 blocks but more than 2^31
    positions): the schedule kernel switches from 32-bit to 64-bit
    positions at 2^31.  Schedule only: the decode itself is not run at
    these lengths."""
    import torch as T
    from mla_paged_kv_metadata_amd import get_mla_metadata
    if last_blocks is not None:
        n = np.full(units, (1 << 25) - 3, dtype=np.int64)
        n[-1] = last_blocks
        assert int(n.sum()) + 2 * units - (1 << 31) == last_blocks - 62
    else:
        n = np.full(units, ((1 << 31) - units) // units, dtype=np.int64)
        assert n.sum() < (1 << 31) <= n.sum() + 2 * units
    sl = (64 * n).astype(np.int32)
    sl[3] -= 17                          # a partial last block
    log(f"cost line near 2^31: {units} units, {int(n.sum()) + 2 * units} positions")
    for P in (8, 1000, 2048):
        md = get_mla_metadata(T.from_numpy(sl).cuda(), 16, 1, num_parts=P)
        T.cuda.synchronize()
        want_md, want_ns = _schedule_by_positions(n, P, 2, sl)
        assert np.array_equal(md.tile_metadata.cpu().numpy(), want_md), P
        assert np.array_equal(md.num_splits.cpu().numpy(), want_ns), P


@pytest.mark.parametrize("topk", [2048, 1001, 200])
def test_sparse_schedule_finds_last_valid_entry_anywhere(topk):
    """Block counts of sparse units whose last valid entry lies in the last
    256 entries of the row, just before them, at the very start, or nowhere,
    for 16-byte-multiple rows, other rows and rows shorter than 256."""
    from oracle import splitkv_schedule as S
    import torch as T
    from mla_paged_kv_metadata_amd import get_mla_metadata
    rng = np.random.default_rng(91 + topk)
    ends = [topk - 1, topk - 256, topk - 257, topk // 2, 1, 0, -1]   # last valid position (-1: none)
    ends = [e for e in ends if e < topk]
    b, s_q = len(ends), 2
    sl = rng.integers(3000, 9000, size=b).astype(np.int32)
    ind = np.full((b, s_q, topk), -1, dtype=np.int32)
    for i, e in enumerate(ends):
        L = int(sl[i])
        for s in range(s_q):
            row = rng.integers(0, L, size=topk).astype(np.int32)
            # past the last valid position: masked entries, -1 or >= L
            tail = np.arange(topk) > e
            row[tail] = np.where(rng.random(int(tail.sum())) < 0.5, -1, L + rng.integers(0, 50, int(tail.sum())))
            ind[i, s] = row
    log(f"sparse schedule topk={topk} ends={ends}")
    nb = S.unit_blocks_sparse(sl, ind)
    want = [max(1, (e + 1 + 63) // 64) for e in ends]
    assert list(nb[::s_q]) == want   # the oracle's own count, by construction
    for P in (8, 40):
        md = get_mla_metadata(T.from_numpy(sl).cuda(), s_q * 16, 1, s_q=s_q, indices=T.from_numpy(ind).cuda(),
                              num_parts=P)
        T.cuda.synchronize()
        ref_md, ref_ns = S.schedule(nb, P, 2, unit_len=np.repeat(sl, s_q))
        assert np.array_equal(md.tile_metadata.cpu().numpy(), ref_md), P
        assert np.array_equal(md.num_splits.cpu().numpy(), ref_ns), P


@pytest.mark.parametrize("fmt", [0, 1])
def test_sparse_prefill_shape(oracle_mod, fmt):
    """Many query tokens per sequence, each with its own top-k list drawn
    from its causal window (prefill), against the oracle on every row."""
    cfg = gen.small_config(2, 48, 128, [600, 1000], causal=True, fmt=fmt, topk=256, seed=61,
                           topk_in_window=True)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=1)
    log(f"sparse prefill fmt={fmt}")
    for parts in (None, 24):
        o, l, _ = run_gpu(inp, num_parts=parts)
        ro, rl = oracle_mod.decode(inp)
        compare(o, l, ro, rl, fmt, f"sparse prefill fmt={fmt} parts={parts}", inp=inp)


@pytest.mark.parametrize("fmt", [0, 1])
def test_dense_prefill_shape(oracle_mod, fmt):
    """Many query tokens per sequence over the whole causal window (a
    prefill: 64 new tokens after a 536-token prefix, and a sequence made of
    its 64 new tokens only), against the oracle on every row.  With 64
    row tiles the library picks 4 parts (tiles fill the device), and 1 and
    16 parts are forced too."""
    cfg = gen.small_config(2, 64, 128, [600, 64], causal=True, fmt=fmt, seed=62)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=1)
    ro, rl = oracle_mod.decode(inp)
    for parts in (None, 1, 16):
        log(f"dense prefill fmt={fmt} parts={parts}")
        o, l, md = run_gpu(inp, num_parts=parts)
        if parts is None:
            assert md.num_parts < 8
        compare(o, l, ro, rl, fmt, f"dense prefill fmt={fmt} parts={md.num_parts}", inp=inp)


def test_single_key_returns_v_row_bitwise():
    cfg = gen.small_config(3, 1, 16, [1, 1, 1], seed=41)
    inp = gen.make_inputs(cfg, poison=True)
    o, l, _ = run_gpu(inp)
    for b in range(3):
        v = gen.bf16_bits_to_f32(inp.kcache[inp.block_table[b, 0], 0, 0].view(np.uint16))[:512]
        assert np.array_equal(o.reshape(3, 16, 512)[b], np.broadcast_to(v.astype(np.float64), (16, 512)))


def _visible_v(inp, b, keys):
    """V rows (fp64) of logical keys `keys` of sequence b, through the block
    table (bf16 pool)."""
    keys = np.asarray(keys, dtype=np.int64)
    pages = inp.block_table[b, keys >> 6].astype(np.int64)
    rows = inp.kcache.view(np.uint16).reshape(-1, 576)[pages * 64 + (keys & 63)]
    return gen.bf16_bits_to_f32(rows[:, :512]).astype(np.float64)


@pytest.mark.parametrize("h_q", [16, 128])
def test_zero_query_counts_keys(h_q):
    """q = 0: every score is 0, so lse = ln N exactly for N visible keys
    (1e-5 separates N from N + 1 up to 32K keys) and out = the plain mean of
    the visible V rows.  Causal s_q = 2 sees L - 1, then L keys; the lengths
    cover every tail residue mod 64 (and several pages), on both tile
    kernels, with forced splits."""
    seqlens = [64 * (r % 5) + r for r in range(64)] + [1000, 4097]
    cfg = gen.small_config(len(seqlens), 2, h_q, seqlens, causal=True, seed=42)
    inp = gen.make_inputs(cfg, poison=True)
    inp.q[:] = 0
    log(f"zero query h_q={h_q}")
    o, l, _ = run_gpu(inp, num_parts=16)
    l = l.reshape(len(seqlens), 2, h_q)
    o = o.reshape(len(seqlens), 2, h_q, 512)
    for b, L in enumerate(seqlens):
        for s in range(2):
            n = L - 1 + s
            if n <= 0:
                assert np.all(np.isneginf(l[b, s])) and np.all(o[b, s] == 0)
                continue
            assert np.all(np.abs(l[b, s] - np.log(n)) <= 1e-5), (b, s, l[b, s, 0], np.log(n))
            mean = _visible_v(inp, b, np.arange(n)).mean(axis=0)
            assert np.all(np.abs(o[b, s] - mean[None, :]) <= 2e-3 + 2.0 ** -7 * np.abs(mean)[None, :]), (b, s)


@pytest.mark.parametrize("h_q", [16, 128])
def test_zero_query_sparse_counts_valid_entries(h_q):
    """Sparse q = 0 with -1 tails and out-of-range entries: lse = ln(number of
    entries inside [0, L)), out = the mean of their V rows (repeated entries
    counted again)."""
    seqlens = [300, 1, 64, 129, 0]
    topk = 150
    rng = np.random.default_rng(9)
    cfg = gen.small_config(len(seqlens), 1, h_q, seqlens, topk=topk, seed=48)
    inp = gen.make_inputs(cfg, poison=True)
    inp.q[:] = 0
    idx = rng.integers(-3, 400, size=(len(seqlens), 1, topk)).astype(np.int32)
    idx[0, 0, 100:] = -1                 # a -1 tail
    idx[1, 0, :] = -1
    idx[1, 0, 7] = 0                     # the only key of a 1-token sequence
    idx[2, 0, :64] = np.arange(64)
    idx[2, 0, 64:] = 5                   # key 5 repeated
    inp.indices = idx
    log(f"zero query sparse h_q={h_q}")
    o, l, _ = run_gpu(inp, num_parts=16)
    l = l.reshape(len(seqlens), h_q)
    o = o.reshape(len(seqlens), h_q, 512)
    for b, L in enumerate(seqlens):
        keys = idx[b, 0][(idx[b, 0] >= 0) & (idx[b, 0] < L)]
        if keys.size == 0:
            assert np.all(np.isneginf(l[b])) and np.all(o[b] == 0)
            continue
        assert np.all(np.abs(l[b] - np.log(keys.size)) <= 1e-5), (b, keys.size, l[b, 0])
        mean = _visible_v(inp, b, keys).mean(axis=0)
        assert np.all(np.abs(o[b] - mean[None, :]) <= 2e-3 + 2.0 ** -7 * np.abs(mean)[None, :]), b


def test_page_permutation_bitwise():
    cfg = gen.small_config(3, 2, 20, [300, 65, 1000], causal=True, seed=43)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=5)
    o1, l1, _ = run_gpu(inp)
    o2, l2, _ = run_gpu(gen.permute_pages(inp, 5))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_poisoned_slots_do_not_leak(fmt):
    cfg = gen.small_config(3, 1, 16, [37, 130, 200], fmt=fmt, seed=44)
    clean = gen.make_inputs(cfg, poison=False, extra_pages=3)
    dirty = gen.make_inputs(cfg, poison=True, extra_pages=3)
    o1, l1, _ = run_gpu(clean)
    o2, l2, _ = run_gpu(dirty)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_sparse_all_indices_equals_dense(oracle_mod, fmt):
    seqlens = [300, 64, 37, 129]
    cfg = gen.small_config(4, 1, 16, seqlens, fmt=fmt, seed=45)
    dense = gen.make_inputs(cfg, poison=True)
    idx = np.full((4, 1, 320), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        idx[b, 0, :L] = np.arange(L)
    sp = dataclasses.replace(dense, indices=idx)
    od, ld, _ = run_gpu(dense)
    osp, lsp, _ = run_gpu(sp)
    compare(osp, lsp, od, ld, fmt, "sparse-vs-dense")


@pytest.mark.parametrize("h_q", [16, 128])
def test_negative_scale(oracle_mod, h_q):
    cfg = gen.small_config(2, 2, h_q, [700, 129], causal=True, seed=46)
    inp = gen.make_inputs(cfg, poison=True)
    inp = dataclasses.replace(inp, softmax_scale=-inp.softmax_scale)
    o, l, _ = run_gpu(inp, num_parts=8)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, inp.fmt, f"negative scale h_q={h_q}", inp=inp)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
@pytest.mark.parametrize("parts", [None, 3, 40])
def test_wide_tiles_long_sequences(oracle_mod, fmt, parts):
    # 2 x 64 = 128 rows per sequence: the 128-row kernel, many full slices,
    # a ragged last page, and splits that start and end inside a sequence.
    cfg = gen.small_config(3, 2, 64, [5000, 3001, 70], causal=True, fmt=fmt, seed=47)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    o, l, _ = run_gpu(inp, num_parts=parts)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, fmt, f"wide long fmt={fmt} parts={parts}", inp=inp)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_sparse_topk_beyond_table(oracle_mod, fmt):
    # topk 2500 > 1024 resolved rows per table fill: the index table of a
    # unit is refilled while its slices stream; duplicates and invalid
    # entries mixed in.
    cfg = gen.small_config(2, 2, 64, [6000, 2600], causal=True, fmt=fmt, topk=2500, seed=48)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    rng = np.random.default_rng(48)
    mask = rng.random(inp.indices.shape) < 0.1
    inp.indices[mask] = rng.integers(-3, 7000, size=int(mask.sum()))
    for parts in (None, 5):
        o, l, _ = run_gpu(inp, num_parts=parts)
        ro, rl = oracle_mod.decode(inp)
        compare(o, l, ro, rl, fmt, f"sparse topk=2500 fmt={fmt} parts={parts}", inp=inp)



@pytest.mark.parametrize("h_q,s_q,causal", [(16, 1, False), (128, 2, True), (128, 1, False)])
def test_scores_growing_along_the_sequence(oracle_mod, h_q, s_q, causal):
    """Scores that rise by about 0.75 per key (hundreds of log2 units over
    the sequence): the running maximum is overtaken again and again, which
    exercises the rescaling of the 16-row kernel and the second pass of the
    128-row dense kernel."""
    seqlens = [320, 70, 1000]
    cfg = gen.small_config(len(seqlens), s_q, h_q, seqlens, causal=causal, seed=4242 + h_q)
    inp = gen.make_inputs(cfg, poison=True)
    rng = np.random.default_rng(7)
    # q = 1 on every dim (with a little noise); key t of sequence b gets
    # t / 32 added on every dim, so its score grows by about 0.75 per key.
    qf = 1.0 + 0.05 * rng.standard_normal(inp.q.shape).astype(np.float32)
    inp.q[...] = gen.f32_to_bf16_bits(qf)
    rows = inp.kcache.view(np.uint16).reshape(inp.kcache.shape[0], 64, 576)
    for b, L in enumerate(seqlens):
        for t in range(L):
            page = int(inp.block_table[b, t // 64])
            k = gen.bf16_bits_to_f32(rows[page, t % 64]) * 0.2 + t / 32.0
            rows[page, t % 64] = gen.f32_to_bf16_bits(k.astype(np.float32))
    log(f"growing scores h_q={h_q} s_q={s_q} causal={causal}")
    o, l, _ = run_gpu(inp, num_parts=8)
    ro, rl = oracle_mod.decode(inp)
    assert rl.max() - rl.min() > 100, "the test needs widely spread scores"
    compare(o, l, ro, rl, inp.fmt, "growing scores", inp=inp)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
@pytest.mark.parametrize("parts,s_q", [(1, 1), (2, 2)])
def test_narrow_pieces_longer_than_64_pages(oracle_mod, fmt, parts, s_q):
    # 16 or 32 rows per sequence (the 16-row kernel) and one or two parts,
    # so a part walks pieces of up to 141 pages: its per-lane page list is
    # reloaded at 64 and 128 pages; 4160 keys is exactly 65 pages.
    cfg = gen.small_config(3, s_q, 16, [9000, 4160, 33], causal=s_q > 1, fmt=fmt, seed=61 + parts)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=3)
    log(f"narrow long pieces fmt={fmt} parts={parts} s_q={s_q}")
    o, l, _ = run_gpu(inp, num_parts=parts)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, fmt, f"narrow long fmt={fmt} parts={parts} s_q={s_q}", inp=inp)


def test_schedule_built_when_metadata_is_omitted():
    """mla_decode_kvcache without `metadata` builds the step's schedule on
    its own stream: same result, bit for bit, as with the schedule passed."""
    from mla_paged_kv_metadata_amd import get_mla_metadata, mla_decode_kvcache
    from gpu_util import to_device
    cfg = gen.small_config(4, 2, 16, [700, 1, 2048, 129], causal=True, seed=50)
    inp = gen.make_inputs(cfg, poison=True)
    q, k, bt, sl, _ = to_device(inp)
    md = get_mla_metadata(sl, 2 * 16, 1, s_q=2)
    o1, l1 = mla_decode_kvcache(q, k, bt, sl, inp.softmax_scale, True, metadata=md)
    o2, l2 = mla_decode_kvcache(q, k, bt, sl, inp.softmax_scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = __import__("oracle").decode(inp)
    compare(o2.float().cpu().numpy().reshape(-1, 512).astype(np.float64),
            l2.cpu().numpy().reshape(-1).astype(np.float64), ro, rl, gen.FMT_BF16, "default metadata")

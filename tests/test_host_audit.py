"""mla_validate_host_inputs: the audit of the values a decode call takes on
trust (sao.pub FlashMLA overview, 三、动手实践: the sparse kernel does no
input checking), run on host copies with no GPU.  Schedules come from the
oracle's sequential walk; each planted fault must be named."""
import ctypes

import numpy as np
import pytest

import mla_inputs as gen
from oracle import splitkv_schedule as S


@pytest.fixture(scope="module")
def lib():
    from mla_paged_kv_metadata_amd import _lib
    return _lib.load()


def _setup(topk=0, causal=False, s_q=1, seqlens=(700, 1, 333, 0, 2048, 129), P=16):
    from mla_paged_kv_metadata_amd import _lib
    cfg = gen.small_config(len(seqlens), s_q, 16, list(seqlens), causal=causal, topk=topk, seed=31,
                           max_blocks=40)
    inp = gen.make_inputs(cfg, extra_pages=2)
    sl = inp.seqlens.astype(np.int32)
    if topk:
        nb = S.unit_blocks_sparse(sl, inp.indices)
        md, ns = S.schedule(nb, P, 2, unit_len=np.repeat(sl, s_q))
    else:
        md, ns = S.schedule(S.unit_blocks_dense(sl), P, 2, unit_len=sl)
    a = _lib.MlaDecodeArgs()
    a.batch, a.s_q, a.h_q, a.h_kv = len(seqlens), s_q, 16, 1
    a.d_qk, a.d_v, a.page_size = 576, 512, 64
    a.num_pages, a.max_blocks_per_seq = inp.num_pages, inp.block_table.shape[1]
    a.topk, a.kv_format, a.softmax_scale, a.causal, a.num_parts = topk, 0, 1 / 24, int(causal), P
    bufs = dict(sl=sl.copy(), bt=inp.block_table.astype(np.int32).copy(),
                idx=(inp.indices.astype(np.int32).copy() if topk else np.zeros(1, np.int32)),
                md=np.asarray(md, dtype=np.int32).copy(), ns=np.asarray(ns, dtype=np.int32).copy())
    return a, bufs


def _audit(lib, a, b):
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    st = lib.mla_validate_host_inputs(ctypes.byref(a), p(b["sl"]), p(b["bt"]), p(b["idx"]), p(b["md"]),
                                      p(b["ns"]))
    return st, lib.mla_last_error().decode()


@pytest.mark.parametrize("topk,causal,s_q", [(0, False, 1), (0, True, 2), (100, True, 2), (70, False, 1)])
def test_good_inputs_pass(lib, topk, causal, s_q):
    a, b = _setup(topk, causal, s_q)
    assert (b["bt"] == -1).any()
    assert _audit(lib, a, b) == (0, "")


def test_planted_faults_are_named(lib):
    a, b = _setup()
    cases = [
        ("bt", (2, 3), 10 ** 6, "block_table[2][3]"),      # 333 keys: block 3 is needed
        ("bt", (4, 0), -1, "block_table[4][0]"),
        ("sl", (1,), -4, "cache_seqlens[1] = -4"),
        ("sl", (1,), 2 ** 31 - 1, "more than max_blocks_per_seq"),
        ("sl", (0,), 640, "stale"),                        # the schedule has 11 blocks for it
        ("ns", (3,), 99, "num_splits"),
        ("md", (5,), 0, "not written by mla_get_metadata"),
        ("md", (0,), 8, "is for 8 parts"),
        ("md", (8 + 8 * 2 + 1,), 77, "does not continue"),
    ]
    for buf, pos, val, words in cases:
        old = b[buf][pos]
        b[buf][pos] = val
        st, msg = _audit(lib, a, b)
        b[buf][pos] = old
        assert st == -1 and words in msg, (buf, pos, val, msg)
    assert _audit(lib, a, b) == (0, "")
    # a page past the sequence is never read
    b["bt"][2, 6] = 10 ** 6
    assert _audit(lib, a, b) == (0, "")


def test_sparse_pages_of_masked_entries_are_not_needed(lib):
    a, b = _setup(topk=70)
    # sequence 3 has no keys: all its entries are masked, its pages unused
    b["bt"][3, :] = 10 ** 6
    assert _audit(lib, a, b) == (0, "")
    i = np.argwhere((b["idx"][0, 0] >= 0) & (b["idx"][0, 0] < 700))[0, 0]
    blk = int(b["idx"][0, 0, i]) >> 6
    b["bt"][0, blk] = -7
    st, msg = _audit(lib, a, b)
    assert st == -1 and f"block_table[0][{blk}] = -7" in msg, msg


def test_null_host_pointer_is_rejected(lib):
    a, b = _setup()
    p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_validate_host_inputs(ctypes.byref(a), p(b["sl"]), None, None, p(b["md"]), p(b["ns"])) == -1

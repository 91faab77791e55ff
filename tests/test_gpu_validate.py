"""mla_validate_inputs: the synchronous debug audit of the device-resident
inputs.  Good inputs (with -1 in unused block-table entries and masked sparse
indices) pass; each planted fault is named.  Nothing here runs a decode on a
faulty input: the audit only copies the buffers to the host."""
import numpy as np
import pytest
import torch

import mla_inputs as gen
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def _case(fmt=0, topk=0, causal=False, s_q=1, seqlens=(700, 1, 333, 0, 2048, 129), seed=31):
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata
    cfg = gen.small_config(len(seqlens), s_q, 16, list(seqlens), causal=causal, fmt=fmt, topk=topk,
                           seed=seed, max_blocks=40)
    inp = gen.make_inputs(cfg, extra_pages=2)
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, s_q * 16, 1, s_q=s_q, indices=idx, num_parts=16)
    call = DecodeCall(q, k, bt, sl, md, causal=causal, indices=idx)
    return inp, call, (q, k, bt, sl, idx, md)


def _fails(call, words):
    from mla_paged_kv_metadata_amd import MlaError
    with pytest.raises(MlaError) as e:
        call.validate()
    msg = str(e.value)
    for w in words:
        assert w in msg, msg
    return msg


@pytest.mark.parametrize("fmt,topk,causal,s_q", [(0, 0, False, 1), (1, 0, True, 2), (0, 100, True, 2),
                                                 (1, 70, False, 1)])
def test_good_inputs_pass(fmt, topk, causal, s_q):
    log(f"validate good fmt={fmt} topk={topk} causal={causal} s_q={s_q}")
    inp, call, _ = _case(fmt, topk, causal, s_q)
    assert (inp.block_table == -1).any()   # unused entries hold -1
    call.validate()
    call.run()   # and the call it vouched for runs
    torch.cuda.synchronize()


def test_bad_page_of_a_needed_block_is_named():
    log("validate bad needed page")
    inp, call, (q, k, bt, sl, idx, md) = _case()
    bt[2, 3] = k.shape[0]            # sequence 2 has 333 keys: block 3 holds keys 192..255
    _fails(call, ["block_table[2][3]", str(k.shape[0])])
    bt[2, 3] = -5
    _fails(call, ["block_table[2][3]", "-5"])


def test_bad_page_past_the_sequence_is_ignored():
    log("validate bad unneeded page")
    inp, call, (q, k, bt, sl, idx, md) = _case()
    bt[2, 6] = 10 ** 6               # 333 keys use blocks 0..5 only
    call.validate()


def test_sparse_only_visible_indices_need_pages():
    log("validate sparse masked pages")
    from mla_paged_kv_metadata_amd import refresh_mla_metadata
    inp, call, (q, k, bt, sl, idx, md) = _case(topk=100, causal=True, s_q=2)
    # Sequence 0 has 700 keys; with causal masking query 0 sees keys < 699
    # and query 1 keys < 700.  Leave block 10 (keys 640..699) referenced only
    # by key 699 of query 0, which that query cannot see.
    blk = 10
    row = idx[0]
    row[(row // 64) == blk] = -1
    row[0, 0] = 699
    bt[0, blk] = -3
    refresh_mla_metadata(md, sl, idx)   # the schedule depends on the indices
    call.validate()
    # Query 1 can see key 699: now block 10 is needed and its page is named.
    row[1, 0] = 699
    refresh_mla_metadata(md, sl, idx)
    _fails(call, [f"block_table[0][{blk}]", "-3"])


def test_length_beyond_the_block_table_is_named():
    log("validate long sequence")
    inp, call, (q, k, bt, sl, idx, md) = _case()
    sl[1] = 40 * 64 + 1
    _fails(call, ["cache_seqlens[1]", "max_blocks_per_seq"])
    sl[1] = -1
    _fails(call, ["cache_seqlens[1]", "negative"])


def test_stale_schedule_is_named():
    log("validate stale schedule")
    from mla_paged_kv_metadata_amd import refresh_mla_metadata
    inp, call, (q, k, bt, sl, idx, md) = _case()
    sl[0] = 640                     # 11 -> 10 blocks; the schedule still says 11
    _fails(call, ["stale", "unit 0"])
    refresh_mla_metadata(md, sl)
    torch.cuda.synchronize()
    call.validate()


def test_tampered_schedule_is_named():
    log("validate tampered schedule")
    inp, call, (q, k, bt, sl, idx, md) = _case()
    t = md.tile_metadata
    P = int(t[0])
    good = t.clone()
    t[5] = 0
    _fails(call, ["not written by mla_get_metadata"])
    t.copy_(good)
    # Drop the last non-empty part: its blocks are no longer covered.
    rows = t[8:8 + 8 * P].view(P, 8)
    last = int((rows[:, 0] >= 0).nonzero().max())
    rows[last] = torch.tensor([-1, 0, -1, 0, 0, 0, 0, 0], dtype=torch.int32, device=t.device)
    _fails(call, ["tile_metadata"])
    t.copy_(good)
    # A wrong split count.
    ns = md.num_splits
    nsg = ns.clone()
    ns[1:] += 1
    _fails(call, ["num_splits"])
    ns.copy_(nsg)
    call.validate()


def test_schedule_for_another_part_count_is_named():
    log("validate part count")
    from mla_paged_kv_metadata_amd import get_mla_metadata
    inp, call, (q, k, bt, sl, idx, md) = _case()
    other = get_mla_metadata(sl, 16, 1, num_parts=24)
    call.args.tile_metadata = other.tile_metadata.data_ptr()
    call.args.num_splits = other.num_splits.data_ptr()
    call._keep = call._keep + (other,)
    _fails(call, ["24 parts"])


def test_binding_rejects_mismatched_shapes():
    """The Python binding refuses, before anything is launched, tensors whose
    shapes would make the kernels read or write outside them."""
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, refresh_mla_metadata
    log("binding shape checks")
    inp, call, (q, k, bt, sl, idx, md) = _case(topk=100, s_q=2)
    with pytest.raises(ValueError):   # out too small
        DecodeCall(q, k, bt, sl, md, indices=idx, out=torch.empty(1, 2, 16, 512, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):   # lse of the wrong dtype
        DecodeCall(q, k, bt, sl, md, indices=idx, lse=torch.empty(q.shape[:3], dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):   # indices with a smaller top-k than the metadata's
        DecodeCall(q, k, bt, sl, md, indices=idx[:, :, :50].contiguous())
    with pytest.raises(ValueError):
        refresh_mla_metadata(md, sl, idx[:, :, :50].contiguous())
    with pytest.raises(ValueError):   # dense call on sparse metadata
        refresh_mla_metadata(md, sl, None)
    with pytest.raises(ValueError):   # metadata for other heads
        md8 = get_mla_metadata(sl, 2 * 8, 1, s_q=2, indices=idx)
        DecodeCall(q, k, bt, sl, md8, indices=idx)
    with pytest.raises(ValueError):   # cache_seqlens of another batch
        DecodeCall(q, k, bt, sl[:3].contiguous(), md, indices=idx)
    out, lse = call.run()             # the well-formed call still runs
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("h_q,topk,fmt", [(16, 0, 0), (128, 0, 0), (128, 64, 1), (16, 64, 1)])
def test_schedule_header_mismatch_gives_defined_output(h_q, topk, fmt):
    """A decode whose num_parts differs from the schedule's, or whose
    schedule header is not one, reads no key: every row gets out = 0 and
    lse = NaN instead of whatever the buffers held."""
    import ctypes
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, _lib
    log(f"header mismatch h_q={h_q} topk={topk} fmt={fmt}")
    seqlens = [700, 1, 333, 0, 2048, 129]
    cfg = gen.small_config(len(seqlens), 1, h_q, seqlens, fmt=fmt, topk=topk, seed=5, max_blocks=40)
    inp = gen.make_inputs(cfg, extra_pages=2)
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, h_q, 1, s_q=1, indices=idx, num_parts=16)
    call = DecodeCall(q, k, bt, sl, md, indices=idx)
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for how in ("num_parts", "magic"):
        call.out.fill_(7.0)
        call.lse.fill_(3.0)
        if how == "num_parts":
            call.args.num_parts = 8      # the schedule holds 16 parts
        else:
            call.args.num_parts = 16
            md.tile_metadata[5] = 0      # not a schedule header
        _lib.check(lib.mla_decode_kvcache(ctypes.byref(call.args), stream))
        torch.cuda.synchronize()
        assert torch.isnan(call.lse).all(), how
        assert (call.out == 0).all(), how
    # a fresh schedule decodes normally again
    md2 = get_mla_metadata(sl, h_q, 1, s_q=1, indices=idx, num_parts=16)
    call2 = DecodeCall(q, k, bt, sl, md2, indices=idx)
    o, l = call2.run()
    torch.cuda.synchronize()
    assert not torch.isnan(l).any()

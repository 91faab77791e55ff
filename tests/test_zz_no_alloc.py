"""mla_decode_kvcache_noalloc (the entry point for callers that cannot
allocate) against mla_decode_kvcache with a caller's workspace, through the
C ABI: two calls in a row on the library's device scratch, the second with
a smaller input (its stale contents from the first must not matter), each
bit for bit equal to the workspace entry point and within the bf16 / FP8
bounds of the oracle; a call too large for the scratch is refused before
anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import mla_inputs as gen
from gpu_util import compare, log, to_device

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _run_both(inp, parts):
    import oracle
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, _lib
    lib = _lib.load()
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, inp.s_q * inp.h_q, 1, s_q=inp.s_q, indices=idx, num_parts=parts)
    ref = DecodeCall(q, k, bt, sl, md, softmax_scale=inp.softmax_scale, causal=inp.causal, indices=idx)
    ref.run()
    na = DecodeCall(q, k, bt, sl, md, softmax_scale=inp.softmax_scale, causal=inp.causal, indices=idx)
    na.out.fill_(3.0)
    na.lse.fill_(3.0)
    na.args.workspace = None          # ignored by the entry point
    na.args.workspace_bytes = 0
    _lib.check(lib.mla_decode_kvcache_noalloc(ctypes.byref(na.args), _stream()))
    torch.cuda.synchronize()
    assert torch.equal(na.out, ref.out) and torch.equal(na.lse, ref.lse)
    assert int(md.num_splits[-1]) > len(inp.seqlens)     # some unit was split: the scratch was used
    o = na.out.float().cpu().numpy().reshape(-1, 512).astype(np.float64)
    l = na.lse.cpu().numpy().reshape(-1).astype(np.float64)
    ro, rl = oracle.decode(inp)
    compare(o, l, ro, rl, inp.fmt, "no-alloc", inp=inp)


def test_two_calls_in_a_row_second_smaller():
    big = gen.make_inputs(gen.small_config(6, 2, 128, [4000, 1, 2500, 0, 3100, 700], causal=True, seed=71),
                          poison=True)
    log("no-alloc call 1: b6 s_q2 h128 causal, 64 parts")
    _run_both(big, 64)
    small = gen.make_inputs(gen.small_config(3, 1, 16, [900, 64, 300], fmt=gen.FMT_FP8, seed=72), poison=True)
    log("no-alloc call 2: b3 s_q1 h16 fp8, 32 parts")
    _run_both(small, 32)


def test_call_beyond_the_scratch_is_refused():
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, _lib, workspace_bytes
    lib = _lib.load()
    inp = gen.make_inputs(gen.small_config(300, 2, 128, [64] * 300, seed=73))
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, 2 * 128, 1, s_q=2, num_parts=512)
    c = DecodeCall(q, k, bt, sl, md)
    assert workspace_bytes(c.args) > 96 << 20
    c.out.fill_(3.0)
    assert lib.mla_decode_kvcache_noalloc(ctypes.byref(c.args), _stream()) == _lib.MLA_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in lib.mla_last_error()
    torch.cuda.synchronize()
    assert (c.out == 3.0).all()      # nothing was launched

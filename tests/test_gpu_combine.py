"""The log-sum-exp combine kernel on its own: mla_decode_combine over
synthetic partial results written into the workspace, against the oracle's
fp64 merge (lse = log sum_i exp(lse_i), out = sum_i exp(lse_i - lse) o_i),
including pieces and whole rows with lse = -inf.  The merge of num_splits
pieces: topnet.top "Was ist FlashMLA?", "MLA-Metadaten abrufen"."""
import ctypes

import numpy as np
import pytest
import torch

import mla_inputs as gen
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def _align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("h_q,s_q,parts,seqlens", [
    (16, 1, 64, [700, 1, 333, 0, 2048, 129, 5000]),   # 16-row units, up to ~40 pieces
    (128, 1, 16, [3000, 64, 2000]),                    # 128-row units
    (16, 2, 256, [20000, 9000]),                       # more than 64 pieces per unit
])
def test_combine_matches_fp64_merge(h_q, s_q, parts, seqlens):
    import oracle
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, _lib
    log(f"combine h_q={h_q} s_q={s_q} parts={parts}")
    cfg = gen.small_config(len(seqlens), s_q, h_q, seqlens, seed=61)
    inp = gen.make_inputs(cfg)
    q, k, bt, sl, _ = to_device(inp)
    md = get_mla_metadata(sl, s_q * h_q, 1, s_q=s_q, num_parts=parts)
    call = DecodeCall(q, k, bt, sl, md)
    ns = md.num_splits.cpu().numpy()
    units, R = len(seqlens), s_q * h_q
    slots = units + parts
    ob = _align256(slots * R * 1024)
    assert call.workspace.numel() >= ob + slots * R * 4
    rng = np.random.default_rng(7)
    o_bits = gen.f32_to_bf16_bits(rng.standard_normal((slots, R, 512)).astype(np.float32))
    lse = (rng.standard_normal((slots, R)) * 3).astype(np.float32)
    lse[rng.random((slots, R)) < 0.1] = -np.inf        # empty pieces
    split_units = [u for u in range(units) if ns[u + 1] - ns[u] > 1]
    assert split_units
    empty_row = (split_units[0], 3)                    # every piece of this row empty
    lse[ns[empty_row[0]]:ns[empty_row[0] + 1], empty_row[1]] = -np.inf
    ws = call.workspace
    ws[:slots * R * 1024].copy_(torch.from_numpy(o_bits.view(np.uint8).reshape(-1)))
    ws[ob:ob + slots * R * 4].copy_(torch.from_numpy(lse.view(np.uint8).reshape(-1)))
    call.out.fill_(5.0)
    call.lse.fill_(9.0)
    lib = _lib.load()
    _lib.check(lib.mla_decode_combine(ctypes.byref(call.args),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    out = call.out.float().cpu().numpy().reshape(units, R, 512).astype(np.float64)
    got_l = call.lse.cpu().numpy().reshape(units, R).astype(np.float64)
    o_f = gen.bf16_bits_to_f32(o_bits).astype(np.float64)
    n_split = 0
    for u in range(units):
        kk = ns[u + 1] - ns[u]
        if kk <= 1:      # not split: the combine leaves the row alone
            assert np.all(out[u] == 5.0) and np.all(got_l[u] == 9.0)
            continue
        n_split += 1
        ro, rl = oracle.merge_partials(lse[ns[u]:ns[u + 1]], o_f[ns[u]:ns[u + 1]])
        inf = np.isneginf(rl)
        assert np.array_equal(inf, np.isneginf(got_l[u])), u
        assert np.all(out[u][inf] == 0)
        assert np.all(np.abs(got_l[u][~inf] - rl[~inf]) <= 1e-5 + 1e-6 * np.abs(rl[~inf])), u
        # bf16 rounding of the result, fp32 weights
        bound = 2.0 ** -8 * np.abs(ro) + 1e-5 * np.abs(o_f[ns[u]:ns[u + 1]]).max()
        assert np.all(np.abs(out[u] - ro) <= bound), (u, float(np.abs(out[u] - ro).max()))
    assert n_split == len(split_units)
    assert np.isneginf(got_l[empty_row]) and np.all(out[empty_row] == 0)

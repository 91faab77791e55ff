"""The FP8-MFMA variant of the decode (qk_fp8 = 1: the query quantised to
e4m3 per row half at a power-of-two scale, QK^T on the fp8 MFMA; sao.pub
FlashMLA overview, 一、项目速览 and 二、核心功能与架构: FP8 cache, sparse decode).

Its result is the exact decode of the quantised query: compared with the
oracle run on oracle.query_quant.quantize_query(q) at the bf16 bounds, on
small shapes (poisoned unused slots, dense, causal, sparse with masked and
out-of-range entries, forced splits) and on sampled rows of the full-size
FP8 and sparse workloads.  Against the exact oracle (unquantised query) the
full-size workloads are held to a looser bound for the quantisation error:
|out - ref| <= 2e-2 + 2e-2 |ref|, |lse - ref| <= 5e-3."""
import dataclasses

import numpy as np
import pytest

import mla_inputs as gen
from gpu_util import compare, log, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FP8_SCOPE_BOUND = dict(atol=2e-2, rtol=2e-2, lse=5e-3)


def _run(inp, num_parts=None, qk_fp8=True):
    from mla_paged_kv_metadata_amd import get_mla_metadata, mla_decode_kvcache
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, inp.s_q * inp.h_q, 1, s_q=inp.s_q, indices=idx, num_parts=num_parts)
    out, lse = mla_decode_kvcache(q, k, bt, sl, inp.softmax_scale, inp.causal, idx, metadata=md, qk_fp8=qk_fp8)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64).reshape(-1, 512),
            lse.cpu().numpy().astype(np.float64).reshape(-1), md)


def _decode_quantised(oracle_mod, inp, sel=None):
    """The oracle's decode of the query as the FP8-MFMA variant quantises
    it (oracle.query_quant)."""
    from oracle.query_quant import quantize_query
    return oracle_mod.decode(inp, sel=sel, q_f64=quantize_query(inp.q))


@pytest.mark.parametrize("s_q,h_q,topk,causal,parts", [(1, 128, 0, False, 16), (2, 64, 0, True, 24),
                                                       (1, 128, 300, False, 32), (3, 48, 0, True, None)])
def test_equals_decode_of_quantised_query(oracle_mod, s_q, h_q, topk, causal, parts):
    seqlens = [700, 1, 333, 0, 2048, 129]
    cfg = gen.small_config(len(seqlens), s_q, h_q, seqlens, causal=causal, fmt=gen.FMT_FP8, topk=topk, seed=83)
    inp = gen.make_inputs(cfg, poison=True)
    log(f"fp8 query s_q={s_q} h_q={h_q} topk={topk} causal={causal} parts={parts}")
    o, l, _ = _run(inp, parts)
    ro, rl = _decode_quantised(oracle_mod, inp)
    compare(o, l, ro, rl, gen.FMT_FP8, "fp8 query vs quantised-query oracle")


def test_negative_scale_quantises_the_negated_query(oracle_mod):
    cfg = gen.small_config(2, 1, 128, [300, 77], fmt=gen.FMT_FP8, seed=84)
    inp = gen.make_inputs(cfg)
    inp = dataclasses.replace(inp, softmax_scale=-inp.softmax_scale)
    o, l, _ = _run(inp, 8)
    ro, rl = _decode_quantised(oracle_mod, inp)
    compare(o, l, ro, rl, gen.FMT_FP8, "fp8 query, negative scale")


def _sample_rows(inp, n, seed):
    rows = inp.batch * inp.s_q * inp.h_q
    rng = np.random.default_rng(seed)
    pick = {0, rows - 1}
    pick.update(int(x) for x in rng.choice(rows, size=min(n, rows), replace=False))
    return np.array(sorted(pick), dtype=np.int32)


@pytest.mark.parametrize("name,seed", [("fp8", 913), ("sparse", 914)])
def test_full_size_sampled_rows(oracle_mod, name, seed):
    cfg = gen.WORKLOADS[name]
    log(f"fp8 query full-size {cfg.name}")
    inp = gen.make_inputs(cfg)
    o, l, md = _run(inp)
    sel = _sample_rows(inp, 96, seed)
    ro, rl = _decode_quantised(oracle_mod, inp, sel=sel)
    compare(o[sel], l[sel], ro, rl, gen.FMT_FP8, f"{cfg.name} vs quantised-query oracle ({len(sel)} rows)")
    eo, el = oracle_mod.decode(inp, sel=sel)
    import gpu_util
    saved = gpu_util.TOL[gen.FMT_FP8]
    gpu_util.TOL[gen.FMT_FP8] = FP8_SCOPE_BOUND
    try:
        compare(o[sel], l[sel], eo, el, gen.FMT_FP8, f"{cfg.name} vs exact oracle, FP8 bound")
    finally:
        gpu_util.TOL[gen.FMT_FP8] = saved


def test_option_is_refused_where_it_does_not_apply():
    from mla_paged_kv_metadata_amd import MlaError
    cfg = gen.small_config(2, 1, 16, [300, 77], fmt=gen.FMT_FP8, seed=85)
    inp = gen.make_inputs(cfg)
    with pytest.raises(MlaError) as e:
        _run(inp, 8)
    assert "qk_fp8" in str(e.value)

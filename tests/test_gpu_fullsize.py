"""GPU parity at the full benchmark workloads, in the launch configuration
bench.py times (default number of split-KV parts), on sampled query rows
that the oracle computes one by one."""
import numpy as np
import pytest

import mla_inputs as gen
from gpu_util import compare, log, run_gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_metadata_amd as m
    m.load_library()


def _sample_rows(inp, n, seed):
    """n rows: the first and last row, every head of the longest and the
    shortest sequence's first query token, the rest uniform."""
    rows = inp.batch * inp.s_q * inp.h_q
    rng = np.random.default_rng(seed)
    pick = {0, rows - 1}
    for b in (int(np.argmax(inp.seqlens)), int(np.argmin(inp.seqlens))):
        base = b * inp.s_q * inp.h_q
        pick.update(range(base, base + min(inp.h_q, 16)))
    pick.update(int(x) for x in rng.choice(rows, size=min(n, rows), replace=False))
    return np.array(sorted(pick), dtype=np.int32)


@pytest.mark.parametrize("name,seed", [("membound", 901), ("mtp", 902), ("fp8", 903), ("sparse", 904),
                                       ("sparse_prefill", 905), ("dense_prefill", 906)])
def test_full_size_sampled_rows(oracle_mod, name, seed):
    cfg = gen.WORKLOADS[name]
    log(f"full-size {cfg.name}")
    inp = gen.make_inputs(cfg)
    o, l, md = run_gpu(inp)
    sel = _sample_rows(inp, 96, seed)
    ro, rl = oracle_mod.decode(inp, sel=sel)
    compare(o[sel], l[sel], ro, rl, inp.fmt, f"{cfg.name} ({len(sel)} rows, {md.num_parts} parts)", inp=inp, sel=sel)


def test_prefill_split_in_two_combines_every_row(oracle_mod):
    """2048 tokens x 128 heads = 262,144 rows in one sequence, forced into
    two parts: the combine covers more than 65,535 four-row groups."""
    cfg = gen.small_config(1, 2048, 128, [2048], causal=True, seed=907)
    log("prefill split in two")
    inp = gen.make_inputs(cfg)
    o, l, md = run_gpu(inp, num_parts=2)
    assert int(md.num_splits[-1]) == 2   # the sequence is split once
    sel = _sample_rows(inp, 96, 907)
    sel = np.unique(np.concatenate([sel, np.arange(inp.s_q * inp.h_q - 16, inp.s_q * inp.h_q)])).astype(np.int32)
    ro, rl = oracle_mod.decode(inp, sel=sel)
    compare(o[sel], l[sel], ro, rl, inp.fmt, f"prefill split in two ({len(sel)} rows)", inp=inp, sel=sel)


@pytest.mark.parametrize("num_parts", [None, 2])
def test_long_prefill_past_32_bit_byte_offsets(oracle_mod, num_parts):
    """One 32,768-token sequence, causal, 128 heads: 4,194,304 query rows.
    q spans 4.8 GB and, split in two, the second part's partial outputs lie
    beyond byte 2^32 of the workspace, so every row offset must be 64-bit.
    q is drawn on the device (seeded) to keep the host work short; the
    oracle reads q only at the sampled rows, which are copied back."""
    s_q, h_q, L = 32768, 128, 32768
    cfg = gen.small_config(1, 1, h_q, [L], causal=True, seed=908)
    kv = gen.make_inputs(cfg)
    from gpu_util import to_device
    _, k, bt, sl, _ = to_device(kv)
    g = torch.Generator(device="cuda").manual_seed(908)
    q = torch.randn(1, s_q, h_q, 576, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    rows = s_q * h_q
    rng = np.random.default_rng(908)
    sel = {0, 1, 127, 128, rows - 1}
    for edge in (2 ** 31 // 1152, 2 ** 32 // 1152, 2 ** 31 // 1024, rows - 16):
        sel.update(range(edge - 2, min(edge + 14, rows)))
    sel.update(int(x) for x in rng.choice(rows, size=48, replace=False))
    sel = np.array(sorted(sel), dtype=np.int32)
    from mla_paged_kv_metadata_amd import get_mla_metadata, mla_decode_kvcache
    log(f"long prefill s_q={s_q} h_q={h_q} L={L} num_parts={num_parts}")
    md = get_mla_metadata(sl, s_q * h_q, 1, s_q=s_q, num_parts=num_parts)
    out, lse = mla_decode_kvcache(q, k, bt, sl, softmax_scale=kv.softmax_scale, causal=True, metadata=md)
    torch.cuda.synchronize()
    if num_parts == 2:
        assert int(md.num_splits[-1]) == 2
    idx = torch.from_numpy(sel.astype(np.int64)).cuda()
    o = out.reshape(rows, 512)[idx].float().cpu().numpy().astype(np.float64)
    l = lse.reshape(rows)[idx].cpu().numpy().astype(np.float64)
    q_host = np.zeros((1, s_q, h_q, 576), dtype=np.uint16)   # only the sampled rows are read
    q_host.reshape(rows, 576)[sel] = q.reshape(rows, 576)[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    del out, q
    ro, rl = oracle_mod.decode_raw(q_host, kv.kcache, kv.fmt, kv.block_table, kv.seqlens, None,
                                   kv.softmax_scale, True, sel=sel)
    compare(o, l, ro, rl, kv.fmt, f"long prefill ({len(sel)} rows, {md.num_parts} parts)")

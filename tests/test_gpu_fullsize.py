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
    compare(o[sel], l[sel], ro, rl, inp.fmt, f"{cfg.name} ({len(sel)} rows, {md.num_parts} parts)")


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
    compare(o[sel], l[sel], ro, rl, inp.fmt, f"prefill split in two ({len(sel)} rows)")

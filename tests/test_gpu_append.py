"""mla_append_kv against the oracle, byte for byte over the whole pool: every
finite bf16 value at scale 1, random rows over many magnitudes, zero and
denormal groups, skipped and out-of-range slots, both row formats, and a
decode of the appended pool."""
import numpy as np
import pytest
import torch

import mla_inputs as gen
from gpu_util import compare, log, run_gpu, to_device
from oracle import kv_append as A

pytestmark = pytest.mark.gpu


def _pool(rng, pages, fmt):
    rb = A.ROW_BF16 if fmt == 0 else A.ROW_FP8
    return rng.integers(0, 256, size=(pages * 64, rb), dtype=np.uint8)


def _gpu_append(pool, rows_bits, slots, fmt):
    from mla_paged_kv_metadata_amd import append_kv
    pages = pool.shape[0] // 64
    k = torch.from_numpy(pool.copy()).cuda()
    if fmt == 0:
        k = k.view(torch.bfloat16).reshape(pages, 64, 1, 576)
    else:
        k = k.reshape(pages, 64, 1, A.ROW_FP8)
    rows = torch.from_numpy(np.ascontiguousarray(rows_bits).view(np.int16)).view(torch.bfloat16).cuda()
    s = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
    append_kv(rows, s, k)
    torch.cuda.synchronize()
    return k.view(torch.uint8).reshape(pool.shape).cpu().numpy()


def _check(pool, rows_bits, slots, fmt, what):
    got = _gpu_append(pool, rows_bits, slots, fmt)
    want = A.append(pool, rows_bits, slots, fmt)
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} pool rows differ, first {bad[:5].tolist()}"


def _bits(x32):
    return (np.asarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_every_bf16_value_at_unit_scale():
    """Every finite bf16 magnitude up to 448 with both signs, each group
    holding 448 so that its scale is exactly 1 and the codes are the values
    themselves rounded to e4m3fn (all ties and subnormals included)."""
    mags = np.arange(0, 0x43E1, dtype=np.uint32)          # bf16 bits 0 .. 448 (0x43E0)
    vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    per_row = 4 * 127
    n = -(-vals.size // per_row)
    vals = np.concatenate([vals, np.zeros(n * per_row - vals.size, dtype=np.uint16)])
    rows = np.zeros((n, 576), dtype=np.uint16)
    for g in range(4):
        rows[:, 128 * g] = 0x43E0                           # 448
        rows[:, 128 * g + 1:128 * (g + 1)] = vals.reshape(n, 4, 127)[:, g]
    rng = np.random.default_rng(1)
    rows[:, 512:] = rng.integers(0, 0x7F80, size=(n, 64))
    pages = -(-n // 64) + 1
    slots = rng.permutation(pages * 64)[:n].astype(np.int32)
    log(f"append exhaustive: {vals.size} values in {n} rows")
    _check(_pool(rng, pages, 1), rows, slots, 1, "exhaustive bf16 at scale 1")


@pytest.mark.parametrize("fmt", [0, 1])
def test_random_rows_and_slots(fmt):
    rng = np.random.default_rng(10 + fmt)
    n, pages = 700, 16
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x *= (2.0 ** rng.integers(-30, 30, size=(n, 1))).astype(np.float32)   # many magnitudes
    rows = _bits(x)
    rows[3, :128] = 0                                     # all-zero group
    rows[4, 128:256] = 0x8000                             # all negative zeros
    rows[5, 256:384] = rng.integers(1, 0x80, 128)         # denormal bf16 values only
    rows[6, :512] = rng.integers(0x0080, 0x0200, 512) | (rng.integers(0, 2, 512) << 15)  # tiny normals
    rows[:, 512:] = rng.integers(0, 0xFFFF, size=(n, 64)) & 0xFF7F  # any RoPE bits but NaN/inf
    slots = rng.permutation(pages * 64)[:n].astype(np.int32)
    slots[::17] = -1                                      # skipped
    slots[5::29] = pages * 64 + 3                         # past the pool: skipped
    log(f"append random fmt={fmt}")
    _check(_pool(rng, pages, fmt), rows, slots, fmt, f"random fmt={fmt}")


def test_empty_append_and_argument_errors():
    from mla_paged_kv_metadata_amd import append_kv, MlaError
    k = torch.zeros(2, 64, 1, 656, dtype=torch.uint8, device="cuda")
    rows = torch.zeros(0, 576, dtype=torch.bfloat16, device="cuda")
    append_kv(rows, torch.zeros(0, dtype=torch.int32, device="cuda"), k)
    assert int(k.sum()) == 0
    with pytest.raises(ValueError):
        append_kv(torch.zeros(3, 576, dtype=torch.float32, device="cuda"),
                  torch.zeros(3, dtype=torch.int32, device="cuda"), k)


@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_reads_what_append_wrote(oracle_mod, fmt):
    """Build a cache token by token with append_kv, then decode it: the
    result must match the oracle's decode of the oracle-built pool."""
    seqlens = [130, 1, 64, 200]
    cfg = gen.small_config(len(seqlens), 1, 16, seqlens, fmt=fmt, seed=77)
    inp = gen.make_inputs(cfg, extra_pages=1)
    rng = np.random.default_rng(12)
    pool_rows = inp.num_pages * 64
    pool = _pool(rng, inp.num_pages, fmt)
    toks, slots = [], []
    for b, L in enumerate(seqlens):
        for t in range(L):
            toks.append(_bits(rng.standard_normal(576).astype(np.float32)))
            slots.append(int(inp.block_table[b, t // 64]) * 64 + t % 64)
    toks = np.stack(toks)
    slots = np.array(slots, dtype=np.int32)
    got = _gpu_append(pool, toks, slots, fmt)
    want = A.append(pool, toks, slots, fmt)
    assert np.array_equal(got, want)
    inp.kcache = want.reshape(inp.kcache.shape)
    log(f"append then decode fmt={fmt}")
    o, l, _ = run_gpu(inp, num_parts=8)
    ro, rl = oracle_mod.decode(inp)
    compare(o, l, ro, rl, fmt, f"append+decode fmt={fmt}", inp=inp)

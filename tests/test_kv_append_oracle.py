"""Pins for the KV-append oracle (CPU only): its e4m3fn rounding against
torch's own float8_e4m3fn cast (a library conversion that shares nothing
with it), closed forms of the 656-byte row (sao.pub FlashMLA overview,
二、核心功能与架构), and the round trip through the oracle's independent C row
decoder."""
import numpy as np
import pytest
import torch

from oracle import kv_append as A


def torch_e4m3(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_codes_match_torch_on_every_value_and_every_tie():
    table = A._TABLE
    mids = (table[:-1] + table[1:]) / 2          # exact ties between neighbours
    rng = np.random.default_rng(5)
    rand = rng.uniform(-448, 448, 20000)
    tiny = rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000)   # subnormal range and its edge
    v = np.concatenate([table, -table, mids, -mids, rand, tiny, [0.0, -0.0, 448.0, -448.0]])
    v32 = v.astype(np.float32)
    exact = np.concatenate([table, -table, mids, -mids])
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)   # ties are exact in fp32
    got = A.e4m3_code(v32.astype(np.float64))
    assert np.array_equal(got, torch_e4m3(v32))


def test_tie_goes_to_even_code():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code wins
    assert A.e4m3_code(np.array([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A)
    assert A.e4m3_code(np.array([1.1875]))[0] == 0x3A
    # subnormal tie: 1.5 * 2^-9 between 0x01 and 0x02
    assert A.e4m3_code(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    assert A.e4m3_code(np.array([-0.0]))[0] == 0x80


def _row(nope_f32, rope_bits):
    bits = np.empty(576, dtype=np.uint16)
    bits[:512] = (np.asarray(nope_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[512:] = rope_bits
    return bits


def test_row_closed_forms():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(512).astype(np.float32)
    x = A.bf16_bits_to_f32((x.view(np.uint32) >> 16).astype(np.uint16))   # bf16 values
    x[128:256] = 0.0                                  # an all-zero group
    x[256:384] = np.clip(x[256:384], -6.0, 6.0)
    x[300] = -7.0                                     # group 2 has a known maximum
    rope = rng.integers(0, 1 << 16, 64).astype(np.uint16)
    row = A.quantize_row(_row(x, rope))
    scales = row[512:528].view("<f4")
    assert scales[1] == 0.0 and not row[128:256].any()
    assert scales[2] == np.float32(np.float32(7.0) / np.float32(448.0))
    assert row[300] == 0xFE                            # -amax -> -448
    assert np.array_equal(row[528:656].view("<u2"), rope)
    for g in (0, 3):
        amax = np.float32(np.abs(x[128 * g:128 * (g + 1)]).max())
        assert scales[g] == np.float32(amax / np.float32(448.0))


def test_round_trip_through_the_c_decoder(oracle_mod):
    rng = np.random.default_rng(7)
    for trial in range(20):
        x = (rng.standard_normal(512) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        x = A.bf16_bits_to_f32((x.view(np.uint32) >> 16).astype(np.uint16))
        rope = rng.integers(0, 0x7F80, 64).astype(np.uint16)   # finite bf16 patterns
        row = A.quantize_row(_row(x, rope))
        dec = oracle_mod.decode_row(row, 1)
        for g in range(4):
            xs = x[128 * g:128 * (g + 1)].astype(np.float64)
            scale = float(row[512:528].view("<f4")[g])
            # half a step of e4m3 at the value's binade, or half the subnormal step
            step = np.where(np.abs(xs) / scale >= 2.0 ** -6,
                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(xs) / scale, 2.0 ** -6))) - 3),
                            2.0 ** -9)
            err = np.abs(dec[128 * g:128 * (g + 1)] - xs)
            assert np.all(err <= 0.5 * step * scale * (1 + 1e-6) + 1e-30), (trial, g, err.max())
        assert np.array_equal(dec[512:], A.bf16_bits_to_f32(rope).astype(np.float64))


def test_append_writes_only_valid_slots():
    rng = np.random.default_rng(8)
    pool = rng.integers(0, 256, size=(3 * 64, A.ROW_FP8), dtype=np.uint8)
    rows = rng.integers(0, 0x7F80, size=(4, 576)).astype(np.uint16)   # finite bf16 patterns
    slots = np.array([5, -1, 3 * 64, 70], dtype=np.int32)
    out = A.append(pool, rows, slots, 1)
    changed = np.nonzero((out != pool).any(axis=1))[0].tolist()
    assert changed == [5, 70]
    assert np.array_equal(out[5], A.quantize_row(rows[0]))
    pool16 = rng.integers(0, 256, size=(64, A.ROW_BF16), dtype=np.uint8)
    out16 = A.append(pool16, rows[:1], np.array([9]), 0)
    assert np.array_equal(out16[9].view("<u2"), rows[0])

"""Pins for the oracle's value decoders (CPU only).

The FP8 cache row (sao.pub FlashMLA overview, 二、核心功能与架构) is 512 FP8
NoPE values, 4 FP32 scales (one per 128 values) and 64 BF16 RoPE values; the
FP8 type is float8_e4m3fn (same page, 四、进阶玩法).  The oracle decodes these
bytes itself; here it is checked against torch's own float8_e4m3fn and
bfloat16 conversions, which share nothing with it, and against closed forms
of the OCP E4M3 format.
"""
import json
import os

import numpy as np
import pytest
import torch

import mla_inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_all_codes_match_torch(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3_to_double(c) for c in range(256)])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert nan_ref.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])


def test_e4m3_closed_forms(oracle_mod):
    e = oracle_mod.e4m3_to_double
    assert e(0x7E) == 448.0          # largest finite: 1.75 * 2^8
    assert e(0xFE) == -448.0
    assert e(0x01) == 2.0 ** -9      # smallest subnormal
    assert e(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert e(0x08) == 2.0 ** -6      # smallest normal
    assert e(0x38) == 1.0            # exponent field 7 = bias
    assert e(0x00) == 0.0 and e(0x80) == 0.0 and np.signbit(e(0x80))


def test_bf16_widening_matches_torch(oracle_mod):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=2000, dtype=np.int64).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # skip inf/nan patterns
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_mod.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(ref, got)


def test_fp8_row_layout_golden():
    """Byte layout facts from the page, stored with their citation."""
    with open(os.path.join(GOLDEN, "fp8_row_layout.json")) as f:
        g = json.load(f)
    assert g["nope_values"] * g["nope_bytes_each"] + g["scales"] * 4 + g["rope_values"] * 2 == gen.FP8_ROW_BYTES
    assert g["nope_values"] // g["scales"] == g["values_per_scale"] == 128
    assert g["page_tokens"] == gen.PAGE


def test_decode_row_fp8_matches_torch_decode(oracle_mod):
    rng = np.random.default_rng(1)
    n = 64
    src = rng.standard_normal((n, 576), dtype=np.float32) * rng.uniform(0.01, 30, size=(n, 1)).astype(np.float32)
    src[3, 128:256] = 0.0  # an all-zero group: scale 0, codes 0
    rows = gen.quantize_fp8_rows(src[:, :512], gen.f32_to_bf16_bits(src[:, 512:]))
    for i in range(n):
        r = rows[i]
        codes = torch.from_numpy(r[:512].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        scales = r[512:528].copy().view("<f4").astype(np.float64)
        rope = torch.from_numpy(r[528:].copy().view("<i2")).view(torch.bfloat16).to(torch.float64).numpy()
        ref = np.concatenate([codes * np.repeat(scales, 128), rope])
        got = oracle_mod.decode_row(r, gen.FMT_FP8)
        assert np.array_equal(ref, got)
        # quantisation error bound of e4m3 (3 mantissa bits, round to nearest):
        # |x - q| <= 2^-4 * |x| for normal codes, <= scale * 2^-10 below them
        x = src[i, :512].astype(np.float64)
        s = np.repeat(scales, 128)
        err = np.abs(got[:512] - x)
        assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6) + 1e-30)
    assert np.all(rows[3, 128:256] == 0) and rows[3, 512 + 4:512 + 8].view("<f4")[0] == 0.0


def test_decode_row_bf16_matches_torch(oracle_mod):
    rng = np.random.default_rng(2)
    bits = gen.f32_to_bf16_bits(rng.standard_normal(576, dtype=np.float32))
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle_mod.decode_row(bits.view(np.uint8), gen.FMT_BF16)
    assert np.array_equal(ref, got)


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000, dtype=np.float32) * 100
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(x), ref)


def test_generator_block_tables_are_valid():
    """Every sequence's blocks map to distinct pool pages, unused entries
    hold -1, and the pages in use cover exactly the needed ones."""
    for seed, (lens, extra) in enumerate([([37, 130], 0), ([1, 64, 65, 700, 0], 3), ([4096] * 3, 1)]):
        cfg = gen.small_config(len(lens), 1, 16, lens, seed=300 + seed, max_blocks=80)
        inp = gen.make_inputs(cfg, extra_pages=extra)
        need = [(L + 63) // 64 for L in lens]
        used = []
        for b, n in enumerate(need):
            row = inp.block_table[b]
            assert np.all(row[n:] == -1)
            assert np.all((row[:n] >= 0) & (row[:n] < inp.num_pages))
            used.extend(row[:n].tolist())
        assert len(set(used)) == len(used) == sum(need)
        assert inp.num_pages == sum(need) + extra

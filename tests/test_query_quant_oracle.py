"""Pins of the query quantisation of the FP8-MFMA variant
(oracle/query_quant.py) against torch's float8_e4m3fn cast and closed
forms (CPU)."""
import numpy as np
import torch

import mla_inputs as gen
from oracle.query_quant import query_codes, quantize_query


def _vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _random_q(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x[:, :256] *= np.exp(rng.uniform(-6, 6, size=(n, 1))).astype(np.float32)   # per-row magnitudes
    x[:, 256:512] *= np.exp(rng.uniform(-6, 6, size=(n, 1))).astype(np.float32)
    return gen.f32_to_bf16_bits(x)


def test_matches_torch_e4m3fn_at_the_power_of_two_scale():
    q = _random_q(300, 1)
    qq = query_codes(q)[0]
    v = _vals(q)
    for h in range(2):
        half = v[:, 256 * h:256 * h + 256]
        amax = np.abs(half).max(axis=1)
        p = np.floor(np.log2(amax)) - 7
        s = 2.0 ** p
        assert np.all(np.abs(half) / s[:, None] < 256)
        ref = torch.from_numpy(half / s[:, None]).to(torch.float8_e4m3fn).to(torch.float64).numpy() * s[:, None]
        assert np.array_equal(qq[:, 256 * h:256 * h + 256], ref)
    assert np.array_equal(qq[:, 512:], v[:, 512:])       # RoPE kept


def test_closed_forms():
    x = np.zeros((4, 576), dtype=np.float32)
    x[0, :512] = 1.0                     # representable: unchanged
    x[1, 3] = 3.0
    x[1, 7] = 1.0 + 1 / 16               # 1.0625 -> ties to even -> 1.0
    x[1, 9] = 1.0 + 3 / 16               # 1.1875 -> ties to even -> 1.25
    x[2, 300] = -5.5
    x[2, 0] = 0.0                        # an all-zero half stays zero
    x[3, 511] = 2.0 ** -100
    q = gen.f32_to_bf16_bits(x)
    qq = query_codes(q)[0]
    assert np.all(qq[0, :512] == 1.0)
    assert qq[1, 3] == 3.0 and qq[1, 7] == 1.0 and qq[1, 9] == 1.25
    assert qq[2, 300] == -5.5 and not np.any(qq[2, :256])
    assert qq[3, 511] == 2.0 ** -100


def test_relative_error_at_most_one_sixteenth():
    q = _random_q(200, 2)
    v, qq = _vals(q), query_codes(q)[0]
    nope_v, nope_q = v[:, :512], qq[:, :512]
    big = np.abs(nope_v) >= np.abs(nope_v).max(axis=1, keepdims=True) * 2.0 ** -13   # normal e4m3 range
    assert np.all(np.abs(nope_q - nope_v)[big] <= 2.0 ** -4 * np.abs(nope_v)[big])


def test_alpha_makes_the_error_orthogonal_to_the_query():
    """(q' - q) . q = 0 per half; alpha = 1 where the codes are exact; a
    zero half stays zero; RoPE kept."""
    q = _random_q(100, 3)
    v, qa = _vals(q), quantize_query(q)
    for h in range(2):
        sl = slice(256 * h, 256 * h + 256)
        err = ((qa[:, sl] - v[:, sl]) * v[:, sl]).sum(axis=1)
        assert np.all(np.abs(err) <= 1e-12 * (v[:, sl] ** 2).sum(axis=1))
    assert np.array_equal(qa[:, 512:], v[:, 512:])
    x = np.zeros((1, 576), dtype=np.float32)
    x[0, :512] = np.tile([1.0, -0.5, 3.0, 0.0], 128)
    qx = quantize_query(gen.f32_to_bf16_bits(x))
    assert np.array_equal(qx[0, :512], x[0, :512].astype(np.float64))
    assert not np.any(quantize_query(np.zeros((1, 576), dtype=np.uint16)))

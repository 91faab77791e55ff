"""Helpers for the GPU tests: move generated inputs to the device, run the
library, and compare with the oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mla_inputs as gen

# Elementwise bounds: |out - ref| <= ATOL + RTOL * |ref|, |lse - ref| <= LSE_TOL.
# bf16 KV: the bound the task states.  FP8 KV against the exact oracle: the
# library rounds each dequantised NoPE value (fp32 code * scale) to bf16
# before the bf16 MFMAs (relative error <= 2^-9 per value), which moves the
# score of key t for row r by at most
#     D_r = |sigma| * 2^-9 * (1 + 2^-15) * max_t sum_{d<512} |q_rd| |k_td|
# over the keys the row sees; lse then moves by at most D_r and out by at
# most (2^-9 + exp(2 D_r) - 1) * max |v| over those keys.  These per-row
# terms (fp8_rounding_terms) are added to the fixed FP8 bounds below.  A
# second comparison takes the same rounding on the oracle's side
# (kernel_precision_pool) and holds the result to the bf16 bounds.
TOL = {
    gen.FMT_BF16: dict(atol=1e-2, rtol=1e-2, lse=1e-3),
    gen.FMT_FP8: dict(atol=2e-2, rtol=2e-2, lse=5e-3),
}

_E4M3 = None


def _e4m3_table() -> np.ndarray:
    global _E4M3
    if _E4M3 is None:
        import oracle
        _E4M3 = np.array([oracle.e4m3_to_double(c) for c in range(256)], dtype=np.float64)
    return _E4M3


def _fp8_nope(rows_u8: np.ndarray) -> np.ndarray:
    """Exact NoPE values (fp64) of 656-byte rows [n, 656]."""
    codes = _e4m3_table()[rows_u8[:, :512]]
    scales = np.ascontiguousarray(rows_u8[:, 512:528]).view("<f4").astype(np.float64)
    return (codes.reshape(-1, 4, 128) * scales[:, :, None]).reshape(-1, 512)


def kernel_precision_pool(inp: gen.Inputs) -> np.ndarray:
    """The FP8 pool as the kernels compute with it, as a bf16 pool
    (uint8 [pages, 64, 1, 1152]): each NoPE value code * scale in fp32,
    rounded to bf16 (nearest, ties to even); RoPE values as stored."""
    rows = inp.kcache.reshape(-1, gen.row_bytes(gen.FMT_FP8))
    codes = _e4m3_table()[rows[:, :512]].astype(np.float32)
    scales = np.ascontiguousarray(rows[:, 512:528]).view("<f4")
    with np.errstate(invalid="ignore", over="ignore"):
        v = (codes.reshape(-1, 4, 128) * scales[:, :, None]).astype(np.float32).reshape(-1, 512)
    u = v.view(np.uint32)
    nope = np.where(np.isnan(v), (u >> 16) | 0x40, (u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    pool = np.empty((rows.shape[0], 576), dtype=np.uint16)
    pool[:, :512] = nope
    pool[:, 512:] = np.ascontiguousarray(rows[:, 528:656]).view("<u2")
    return pool.view(np.uint8).reshape(inp.num_pages, 64, 1, 1152)


def fp8_rounding_terms(inp: gen.Inputs, sel=None):
    """Per row (flat index (b s_q + s) h_q + h, all or `sel`): D_r and
    max |v| over the keys the row sees (see the bounds above)."""
    B, S, H = inp.batch, inp.s_q, inp.h_q
    rows_all = np.arange(B * S * H) if sel is None else np.asarray(sel)
    pool = inp.kcache.reshape(-1, gen.row_bytes(gen.FMT_FP8))
    qn = np.abs(gen.bf16_bits_to_f32(inp.q.reshape(-1, gen.D_QK)[:, :512]).astype(np.float64))
    delta = np.zeros(rows_all.size)
    vmax = np.zeros(rows_all.size)
    groups = {}
    for i, r in enumerate(rows_all.tolist()):
        groups.setdefault(r // H, []).append(i)
    for bs, idx in groups.items():
        b, s = divmod(bs, S)
        L = int(inp.seqlens[b])
        W = min(max(L - S + 1 + s, 0), L) if inp.causal else L
        if inp.indices is None:
            t = np.arange(W)
        else:
            t = inp.indices[b, s]
            t = t[(t >= 0) & (t < W)]
        if t.size == 0:
            continue
        prow = inp.block_table[b, t >> 6].astype(np.int64) * 64 + (t & 63)
        k = np.abs(_fp8_nope(pool[prow]))
        rr = rows_all[idx]
        dots = k @ qn[rr].T                       # [keys, rows]
        delta[idx] = abs(inp.softmax_scale) * 2.0 ** -9 * (1 + 2.0 ** -15) * dots.max(axis=0)
        vmax[idx] = k.max()
    return delta, vmax


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: gen.Inputs, device="cuda"):
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(device)
    if inp.fmt == gen.FMT_BF16:
        k = torch.from_numpy(inp.kcache.view(np.int16)).view(torch.bfloat16)
        k = k.reshape(inp.num_pages, 64, 1, 576).to(device)
    else:
        k = torch.from_numpy(inp.kcache).to(device)
    bt = torch.from_numpy(inp.block_table).to(device)
    sl = torch.from_numpy(inp.seqlens).to(device)
    idx = torch.from_numpy(inp.indices).to(device) if inp.indices is not None else None
    return q, k, bt, sl, idx


def run_gpu(inp: gen.Inputs, num_parts=None, dev_tensors=None):
    from mla_paged_kv_metadata_amd import get_mla_metadata, mla_decode_kvcache
    q, k, bt, sl, idx = dev_tensors if dev_tensors is not None else to_device(inp)
    md = get_mla_metadata(sl, inp.s_q * inp.h_q, 1, s_q=inp.s_q, indices=idx, num_parts=num_parts)
    out, lse = mla_decode_kvcache(q, k, bt, sl, metadata=md, softmax_scale=inp.softmax_scale,
                                  causal=inp.causal, indices=idx)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    l = lse.cpu().numpy().astype(np.float64).reshape(-1)
    return o, l, md


def compare(o, l, ro, rl, fmt, what="", inp=None, sel=None):
    """Assert the GPU result matches the oracle within the bounds.  For FP8
    pools pass the inputs (and the selected rows): the per-row rounding
    terms are added, and the result is also held to the bf16 bounds against
    the oracle run on the kernel-precision pool."""
    t = dict(TOL[fmt])
    if fmt == gen.FMT_FP8 and inp is not None:
        import oracle
        eo, el = oracle.decode_raw(inp.q, kernel_precision_pool(inp), gen.FMT_BF16, inp.block_table,
                                   inp.seqlens, inp.indices, inp.softmax_scale, inp.causal, sel=sel)
        compare(o, l, eo, el, gen.FMT_BF16, what + " (kernel precision)")
        delta, vmax = fp8_rounding_terms(inp, sel)
        t["lse"] = t["lse"] + delta
        t["atol"] = t["atol"] + ((2.0 ** -9 + np.expm1(2 * delta)) * vmax)[:, None]
    inf_ref = np.isinf(rl)
    assert np.array_equal(inf_ref, np.isinf(l)), f"{what}: -inf lse pattern differs"
    assert np.all(rl[inf_ref] < 0) and np.all(l[inf_ref] < 0)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    fin = ~inf_ref
    dl = np.abs(l[fin] - rl[fin])
    do = np.abs(o - ro)
    bound = t["atol"] + t["rtol"] * np.abs(ro)
    worst = float((do / bound).max()) if do.size else 0.0
    rel_rms = float(np.linalg.norm(o - ro) / max(np.linalg.norm(ro), 1e-30))
    log(f"  {what}: max|dlse|={dl.max() if dl.size else 0:.3e} max|dout|={do.max():.3e} "
        f"worst/bound={worst:.3f} relRMS={rel_rms:.2e}")
    lse_tol = np.broadcast_to(np.asarray(t["lse"], dtype=np.float64), rl.shape)[fin]
    assert np.all(dl <= lse_tol), f"{what}: lse error {dl.max()} (worst ratio {float((dl / lse_tol).max())})"
    assert np.all(do <= bound), f"{what}: out error beyond bound (worst ratio {worst})"
    assert np.all(o[inf_ref] == 0), f"{what}: empty rows must be zero"
    return rel_rms

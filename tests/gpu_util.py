"""Helpers for the GPU tests: move generated inputs to the device, run the
library, and compare with the oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mla_inputs as gen

# Elementwise bounds: |out - ref| <= ATOL + RTOL * |ref|, |lse - ref| <= LSE_TOL.
# bf16 KV: the bound the task states.  FP8 KV, against the oracle on the
# exact stored values (code * scale in fp64): the scores take every e4m3
# code exactly and the fp32 group scales after the MFMAs, so no product
# code * scale is rounded there; for PV the 16-row kernel scales the
# probabilities of each V group and the 128-row kernels round code * scale
# to bf16, a rounding the bf16 path has anyway (its V is bf16), so the bf16
# bounds apply unchanged.
TOL = {
    gen.FMT_BF16: dict(atol=1e-2, rtol=1e-2, lse=1e-3),
    gen.FMT_FP8: dict(atol=1e-2, rtol=1e-2, lse=1e-3),
}


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
    """Assert the GPU result matches the oracle within the bounds of TOL
    (inp and sel are accepted for callers that pass them; the bounds need
    neither)."""
    t = dict(TOL[fmt])
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

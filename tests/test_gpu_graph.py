"""The decode step (schedule + split-KV kernel + combine) captured in a HIP
graph and replayed: every replay must equal the eager result bit for bit,
with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import mla_inputs as gen
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h_q,fmt,topk", [(16, 0, 0), (128, 0, 0), (16, 1, 0), (128, 1, 100),
                                          (16, 0, 200), (128, 1, 0), (128, 0, 100)])
def test_graph_replay_matches_eager(h_q, fmt, topk):
    from mla_paged_kv_metadata_amd import DecodeCall, get_mla_metadata, refresh_mla_metadata
    seqlens = [700, 1, 333, 0, 2048, 129]
    cfg = gen.small_config(len(seqlens), 1, h_q, seqlens, causal=False, fmt=fmt, topk=topk, seed=900 + h_q)
    inp = gen.make_inputs(cfg, poison=True, extra_pages=2)
    log(f"graph case h_q={h_q} fmt={fmt} topk={topk}")
    q, k, bt, sl, idx = to_device(inp)
    md = get_mla_metadata(sl, inp.s_q * inp.h_q, 1, s_q=inp.s_q, indices=idx, num_parts=16)
    call = DecodeCall(q, k, bt, sl, md, softmax_scale=inp.softmax_scale, causal=inp.causal, indices=idx)

    def step():
        refresh_mla_metadata(md, sl, idx)
        call.partial()
        call.combine()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_o, ref_l = call.out.clone(), call.lse.clone()
    ref_md, ref_ns = md.tile_metadata.clone(), md.num_splits.clone()
    assert int(md.num_splits[-1]) > len(seqlens), "some units must be split"

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        # eager work in between: clobber the outputs and the schedule
        call.out.fill_(0)
        call.lse.fill_(0)
        md.tile_metadata.fill_(-7)
        md.num_splits.fill_(-7)
        call.workspace.fill_(255)   # NaN partials: the combine must see this replay's
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(md.tile_metadata, ref_md) and torch.equal(md.num_splits, ref_ns), f"replay {r}: schedule"
        assert torch.equal(call.out, ref_o), f"replay {r}: out differs from eager"
        assert torch.equal(call.lse, ref_l), f"replay {r}: lse differs from eager"
        # and the eager path still agrees after a replay
        step()
        torch.cuda.synchronize()
        assert torch.equal(call.out, ref_o) and torch.equal(call.lse, ref_l)

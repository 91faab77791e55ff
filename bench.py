#!/usr/bin/env python3
"""Benchmark of MLA paged-KV decoding on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = one pass of the whole decode path over one batch: the split-KV
schedule (mla_get_metadata), the split-KV attention kernel and the combine
kernel, enqueued on one stream.  The workload is the memory-bound
variable-length decode (batch 64, 1 query token, 16 heads, lengths uniform
in [1, 8192], bf16 pages); `value` is its KV-read bandwidth (algorithmic KV
bytes / step time).  The compute-bound MTP decode (batch 128, 2 query
tokens, 128 heads, L = 4096, causal) is timed the same way and reported in
bf16 TFLOPS under "mtp"; the FP8 and sparse workloads under "fp8"/"sparse".

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Six physical copies of each page pool (same logical cache, pages shuffled
differently; --replicas) are used in rotation so that consecutive steps do
not hit the 256 MB Infinity Cache.

Timed loops per workload:
  * the steps replayed from HIP graphs, as a serving loop runs them: one
    graph holds four rotations of consecutive steps (one step per pool copy,
    each step complete: schedule, split-KV kernel, combine), so the launch
    overhead of a graph is shared by 24 steps; wall time per step gives
    `value` / `ms_per_step`.  Every graph's output is checked bit for bit
    against an eager step first.
  * the split-KV kernel alone, replayed from a graph of back-to-back
    launches (one per pool copy) with HIP events on the launch stream
    around the replays: its mean launch duration gives the roofline's
    `achieved` (algorithmic bytes or flops per launch over it).
  * the same step launched eagerly with HIP events around each kernel
    (timing_ms: per-kernel event times, which include dispatch latency).
`roofline.traffic` (measured HBM bytes per launch) is read from the
committed counter summary in profiles/ when it was taken on the kernel
sources as they are now, else null.

    python bench.py --pmc-run [membound|mtp|fp8|sparse]

runs the workload that the counter summaries are taken on: for the
memory-bound one a plain fp32 copy of known size first (the counters'
calibration), then a few eager steps.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
GRAPH_ROTATIONS = 4            # rotations of the pool copies in one graph of the timed loop


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(inp) -> dict:
    """What the decode must move once: KV rows it attends to, q, out, lse and
    the block-table entries it uses."""
    import mla_inputs as gen
    kv = inp.kv_bytes_read()
    rows = inp.batch * inp.s_q * inp.h_q
    n_blocks = int(sum((int(L) + 63) // 64 for L in inp.seqlens))
    other = rows * (gen.D_QK * 2 + gen.D_V * 2 + 4) + 4 * n_blocks
    if inp.indices is not None:
        other += inp.indices.size * 4
    return {"kv": kv, "total": kv + other}


class Workload:
    """Device-resident inputs (with pool replicas) and prepared calls."""

    def __init__(self, name: str, replicas: int):
        import torch
        import mla_inputs as gen
        import mla_paged_kv_metadata_amd as m
        self.cfg = gen.WORKLOADS[name]
        t0 = time.time()
        self.inp = gen.make_inputs(self.cfg)
        log(f"[bench] {self.cfg.name}: inputs generated in {time.time() - t0:.1f}s "
            f"({self.inp.num_pages} pages)")
        inp = self.inp
        dev = "cuda"
        self.q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
        self.seqlens = torch.from_numpy(inp.seqlens).to(dev)
        self.indices = torch.from_numpy(inp.indices).to(dev) if inp.indices is not None else None
        # One schedule buffer per pool copy (each step builds its own).
        self.mds = [m.get_mla_metadata(self.seqlens, inp.s_q * inp.h_q, 1, s_q=inp.s_q,
                                       indices=self.indices) for _ in range(replicas)]
        self.md = self.mds[0]
        self.calls = []
        out = lse = ws = None
        for r in range(replicas):
            v = inp if r == 0 else gen.permute_pages(inp, 7919 * r)
            if inp.fmt == gen.FMT_BF16:
                k = torch.from_numpy(v.kcache.view(np.int16)).view(torch.bfloat16).reshape(
                    v.num_pages, 64, 1, 576).to(dev)
            else:
                k = torch.from_numpy(v.kcache).to(dev)
            bt = torch.from_numpy(v.block_table).to(dev)
            c = m.DecodeCall(self.q, k, bt, self.seqlens, self.mds[r], softmax_scale=inp.softmax_scale,
                             causal=inp.causal, indices=self.indices, out=out, lse=lse, workspace=ws)
            out, lse, ws = c.out, c.lse, c.workspace
            self.calls.append(c)
        torch.cuda.synchronize()
        self.bytes = algorithmic_bytes(inp)
        self.flops = inp.flops()

    def step(self, i, ev=None):
        import mla_paged_kv_metadata_amd as m
        c = self.calls[i % len(self.calls)]
        if ev is not None:
            ev[0].record()
        m.refresh_mla_metadata(self.mds[i % len(self.calls)], self.seqlens, self.indices)
        if ev is not None:
            ev[1].record()
        c.partial()
        if ev is not None:
            ev[2].record()
        c.combine()
        if ev is not None:
            ev[3].record()

    def capture(self):
        """HIP graphs holding consecutive whole steps, one step per pool copy
        in rotation: graphs[n] runs steps on copies 0 .. n - 1, so a full
        rotation is one graph launch (as a serving loop launches one graph
        per decode step of many kernels, not one per kernel)."""
        import torch
        import mla_paged_kv_metadata_amd as m
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(2 * len(self.calls)):
                self.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graphs = {}
        for n in range(1, len(self.calls) + 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r, c in enumerate(self.calls[:n]):
                    m.refresh_mla_metadata(self.mds[r], self.seqlens, self.indices)
                    c.partial()
                    c.combine()
            self.graphs[n] = g
        # Several rotations in one graph, so that the GPU idle time of a
        # graph launch is shared by more steps (a serving loop's graph holds
        # the decode step of every layer).
        self.graph_rot = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph_rot):
            for _ in range(GRAPH_ROTATIONS):
                for r, c in enumerate(self.calls):
                    m.refresh_mla_metadata(self.mds[r], self.seqlens, self.indices)
                    c.partial()
                    c.combine()
        # The split-KV kernel alone, once per pool copy, back to back: its
        # launch duration measured without the dispatch latency that HIP
        # events around a single eager launch include.
        self.graph_k2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph_k2):
            for c in self.calls:
                c.partial()
        torch.cuda.synchronize()

    def check_graph(self):
        """Each graph's out/lse must equal the eager step's, bit for bit (all
        pool copies hold the same logical cache, so every step of a graph
        writes the same result)."""
        import torch
        c0 = self.calls[0]
        self.step(0)
        torch.cuda.synchronize()
        ref_o, ref_l = c0.out.clone(), c0.lse.clone()
        checks = list(self.graphs.items()) + [(GRAPH_ROTATIONS * len(self.calls), self.graph_rot)]
        for n, g in checks:
            c0.out.fill_(0)
            c0.lse.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            if not (torch.equal(c0.out, ref_o) and torch.equal(c0.lse, ref_l)):
                raise RuntimeError(f"graph of {n} steps differs from the eager step")

    def _replay_steps(self, steps: int):
        full = len(self.calls)
        big = GRAPH_ROTATIONS * full
        for _ in range(steps // big):
            self.graph_rot.replay()
        rest = steps % big
        for _ in range(rest // full):
            self.graphs[full].replay()
        if rest % full:
            self.graphs[rest % full].replay()

    def time_graph(self, steps: int, warmup: int) -> float:
        import torch
        self._replay_steps(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self._replay_steps(steps)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def time_k2(self, reps: int) -> float:
        """Mean split-KV launch duration (ms) from HIP events on the launch
        stream around replays of the graph of back-to-back launches."""
        import torch
        for _ in range(2):
            self.graph_k2.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            self.graph_k2.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(self.calls))

    def time(self, steps: int, warmup: int) -> dict:
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        md_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
        part_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
        comb_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
        step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
        return {
            "wall_ms_per_step": (t1 - t0) * 1e3 / steps,
            "event_ms_per_step": float(step_ms.mean()),
            "metadata_ms": float(md_ms.mean()),
            "splitkv_ms": float(part_ms.mean()),
            "splitkv_ms_median": float(np.median(part_ms)),
            "combine_ms": float(comb_ms.mean()),
        }


def bench_append(reps: int) -> dict:
    """mla_append_kv: a bulk append of 65,536 tokens, 64 sequences of 1024
    tokens each written to consecutive positions of their own pages, the
    pages scattered over a pool twice that size (FP8 and bf16 rows), and the
    append of one MTP decode step (128 sequences x 2 tokens at random
    positions, FP8).  Algorithmic bytes per token: the 1152-byte input row,
    the 4-byte slot and the written row."""
    import torch
    import mla_paged_kv_metadata_amd as m
    out = {}
    g = torch.Generator(device="cpu").manual_seed(1005)
    for label, n, fmt in (("fp8_65536", 65536, 1), ("bf16_65536", 65536, 0), ("fp8_256", 256, 1)):
        pages = max(2, 2 * n // 64)
        rows = torch.randn(n, 576, generator=g).to(torch.bfloat16).cuda()
        if n >= 1024:   # whole pages of consecutive positions, pages scattered
            page_of = torch.randperm(pages, generator=g)[: n // 64].to(torch.int64)
            slots = (page_of.repeat_interleave(64) * 64 + torch.arange(64).repeat(n // 64)).to(torch.int32).cuda()
        else:
            slots = torch.randperm(pages * 64, generator=g)[:n].to(torch.int32).cuda()
        if fmt == 1:
            k = torch.zeros(pages, 64, 1, 656, dtype=torch.uint8, device="cuda")
        else:
            k = torch.zeros(pages, 64, 1, 576, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            m.append_kv(rows, slots, k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            m.append_kv(rows, slots, k)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        row_out = 656 if fmt == 1 else 1152
        nbytes = n * (1152 + 4 + row_out)
        out[label] = {"tokens": n, "kv_format": "fp8_656" if fmt == 1 else "bf16", "us": round(ms * 1e3, 2),
                      "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del rows, slots, k
    return out


def cpu_baseline(inp, target_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the same workload: whole
    sequences (all their query rows), taken in order until about target_s of
    CPU work; reported as KV-read GB/s over the sampled sequences."""
    import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    # calibrate on the first sequence
    rows_per_b = inp.s_q * inp.h_q
    sel0 = np.arange(rows_per_b, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.decode(inp, sel=sel0, threads=threads)
    t_first = time.perf_counter() - t0
    keys0 = max(int(inp.seqlens[0]), 1)
    per_key = t_first / keys0
    nb = 1
    keys = keys0
    while nb < inp.batch and (keys + int(inp.seqlens[nb])) * per_key < target_s:
        keys += int(inp.seqlens[nb])
        nb += 1
    sel = np.arange(nb * rows_per_b, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.decode(inp, sel=sel, threads=threads)
    dt = time.perf_counter() - t0
    # A sample shorter than the target (the whole workload fits in it) is
    # decoded again until about target_s of CPU work has been timed.
    passes = 1
    if dt < 0.5 * target_s:
        passes = max(1, int(target_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(passes):
            oracle.decode(inp, sel=sel, threads=threads)
        dt = time.perf_counter() - t0
    kv = int(sum(int(inp.seqlens[b]) for b in range(nb))) * (1152 if inp.fmt == 0 else 656)
    return {"value": kv * passes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {nb} of {inp.batch} sequences, all {rows_per_b} query rows each "
                      f"({kv / 1e6:.1f} MB of KV rows), {passes} pass(es) in {dt:.1f} s"}


# The dominant kernel of each workload, as rocprofv3 names it, and the
# sources it is built from (the counter summary is valid while they match).
KERNEL_NAMES = {
    "membound": "void mla::narrow::narrow_kernel<0, false>(mla::DecodeParams)",
    "mtp": "mla::wide::offset_kernel(mla::DecodeParams)",
    "fp8": "void mla::wide::wide_kernel<1, false>(mla::DecodeParams)",
    "sparse": "void mla::wide::wide_kernel<1, true>(mla::DecodeParams)",
    "sparse_prefill": "void mla::wide::wide_kernel<1, true>(mla::DecodeParams)",
    "dense_prefill": "mla::wide::offset_kernel(mla::DecodeParams)",
}
KERNEL_SOURCES = {
    "membound": ["mla_decode_narrow.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "mtp": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "fp8": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "sparse": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "sparse_prefill": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "dense_prefill": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "narrow_kernel_membound_b64_h16_traffic.md")
# Kernel trace + MFMA counter summaries of the compute-bound workloads.
MFMA_FILES = {
    "mtp": os.path.join(ROOT, "profiles", "offset_kernel_mtp_b128_sq2_h128_kernel_stats.md"),
    "fp8": os.path.join(ROOT, "profiles", "wide_kernel_fp8_b64_h128_L8192_kernel_stats.md"),
    "sparse": os.path.join(ROOT, "profiles", "wide_kernel_sparse_b32_h128_top2048_kernel_stats.md"),
    "sparse_prefill": os.path.join(ROOT, "profiles", "wide_kernel_sparse_prefill_sq2048_h128_top2048_kernel_stats.md"),
    "dense_prefill": os.path.join(ROOT, "profiles", "offset_kernel_dense_prefill_sq2048_h128_L8192_kernel_stats.md"),
}


def sources_sha(name: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mla_paged_kv_metadata_amd", "csrc")
    for f in KERNEL_SOURCES[name]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (a line `traffic-json: {...}`), or None if there is none or it
    was taken on other kernel sources."""
    if name != "membound":
        return None
    return _summary_json(TRAFFIC_FILE, "traffic-json", name)


def _summary_json(path: str, tag: str, name: str):
    """The `tag: {...}` line of a committed counter summary, or None if there
    is none or it was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith(tag + ":"):
                d = json.loads(line.split(":", 1)[1])
                return d if d.get("sources_sha") == sources_sha(name) else None
    return None


def measured_mfma(name: str):
    """MFMA counter figures (MfmaUtil, MFMA flops) of the dominant kernel from
    the committed summary, or None."""
    return _summary_json(MFMA_FILES[name], "mfma-json", name) if name in MFMA_FILES else None


def pmc_run(which: str):
    """The run the counter summaries are taken on: for the memory-bound
    workload, first a plain copy of known size (fp32, 256 Mi elements: 1 GiB
    read, 1 GiB written: the counters' calibration), then six eager steps of
    the workload."""
    import torch
    if which == "membound":
        n = 256 * 1024 * 1024
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads n*4 B, writes n*4 B
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log(f"[bench] copy of {n * 4} B x3")
    w = Workload(which, 3)
    for i in range(6):
        w.step(i)
    torch.cuda.synchronize()
    log(f"[bench] pmc run done: 6 steps of {w.cfg.name} ({w.flops} flops per split-KV launch)")


def run_workload(name: str, replicas: int, steps: int, warmup: int):
    import torch
    w = Workload(name, replicas)
    w.capture()
    w.check_graph()
    t = w.time(steps, warmup)
    t["graph_ms_per_step"] = w.time_graph(steps, warmup)
    t["splitkv_ms_eager_events"] = t["splitkv_ms"]
    t["splitkv_ms"] = w.time_k2(max(3, steps // len(w.calls)))
    return w, t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true",
                    help="skip the MTP, FP8 and sparse workloads")
    ap.add_argument("--only", choices=["mtp", "fp8", "sparse", "sparse_prefill", "dense_prefill", "append"],
                    default=None,
                    help="time just this secondary workload (for profiling)")
    ap.add_argument("--pmc-run", nargs="?", const="membound", default=None,
                    choices=["membound", "mtp", "fp8", "sparse", "sparse_prefill", "dense_prefill"],
                    help="the run hardware counters are collected on (no timing)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the decode is measured on one MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_paged_kv_metadata_amd as m
    m.load_library()   # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.pmc_run:
        pmc_run(args.pmc_run)
        return

    if args.only == "append":
        print(json.dumps({"append": bench_append(args.steps)}), flush=True)
        return
    if args.only is not None:
        w, t = run_workload(args.only, args.replicas, args.steps, args.warmup)
        print(json.dumps({"workload": w.cfg.name, "timing_ms": t,
                          "splitkv_tflops": w.flops / (t["splitkv_ms"] * 1e-3) / 1e12}), flush=True)
        return

    prim, tm = run_workload("membound", args.replicas, args.steps, args.warmup)
    log("[bench] membound timed")
    kv = prim.bytes["kv"]
    step_ms = tm["graph_ms_per_step"]
    value = kv / (step_ms * 1e-3) / 1e9
    achieved = prim.bytes["total"] / (tm["splitkv_ms"] * 1e-3) / 1e9
    traffic = measured_traffic("membound")
    result = {
        "metric": "MLA paged decode: KV-read GB/s (h_q=16) and bf16 TFLOPS (h_q=128,s_q=2)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": prim.cfg.name,
            "batch": prim.inp.batch, "s_q": prim.inp.s_q, "h_q": prim.inp.h_q,
            "seqlens": "uniform[1,8192], seed 1001",
            "sum_seqlens": int(prim.inp.seqlens.sum()),
            "kv_bytes": kv, "kv_format": "bf16", "page_size": 64,
            "num_parts": prim.md.num_parts, "pool_replicas": args.replicas,
            "step": f"metadata + split-KV + combine, replayed from HIP graphs of "
                    f"{GRAPH_ROTATIONS * args.replicas} consecutive steps",
        },
        "timing_ms": {k: round(v, 5) for k, v in tm.items()},
        # KV bytes over the decode kernels alone (split-KV + combine, HIP
        # events), the schedule being built once per step for all layers.
        "decode_kv_gbs": round(kv / ((tm["splitkv_ms"] + tm["combine_ms"]) * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": KERNEL_NAMES["membound"],
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic["bytes_per_launch"]),
            "algorithmic_bytes": prim.bytes["total"],
        },
    }
    if traffic is not None:
        result["roofline"]["traffic_detail"] = {k: traffic[k] for k in
                                                ("fetch_bytes", "write_bytes", "fetch_factor", "write_factor")
                                                if k in traffic}
    if not args.only_primary:
        extra = {}
        for key in ("mtp", "fp8", "sparse", "sparse_prefill", "dense_prefill"):
            del prim
            torch.cuda.empty_cache()
            log(f"[bench] timing {key}")
            w, t = run_workload(key, args.replicas, max(10, args.steps // 2), args.warmup)
            step_s = t["graph_ms_per_step"] * 1e-3
            extra[key] = {
                "workload": w.cfg.name,
                "ms_per_step": round(t["graph_ms_per_step"], 5),
                "tflops": round(w.flops / step_s / 1e12, 2),
                "kv_gbs": round(w.bytes["kv"] / step_s / 1e9, 1),
                "splitkv_kernel": KERNEL_NAMES[key],
                "splitkv_ms": round(t["splitkv_ms"], 5),
                "combine_ms": round(t["combine_ms"], 5),
                "metadata_ms": round(t["metadata_ms"], 5),
                "eager_ms_per_step": round(t["wall_ms_per_step"], 5),
                "splitkv_tflops": round(w.flops / (t["splitkv_ms"] * 1e-3) / 1e12, 2),
                "mfma_frac_of_bf16_peak": round(w.flops / (t["splitkv_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "rocprof": measured_mfma(key),
                "flops": w.flops,
                "kv_bytes": w.bytes["kv"],
            }
            prim = w
        log("[bench] timing append")
        extra["append"] = bench_append(max(10, args.steps // 2))
        result["secondary"] = extra
        del prim
    if not args.no_cpu_baseline:
        import mla_inputs as gen
        log("[bench] cpu baseline (oracle)")
        inp = gen.make_inputs(gen.WORKLOADS["membound"])
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

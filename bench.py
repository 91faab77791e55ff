#!/usr/bin/env python3
"""Benchmark of MLA paged-KV decoding on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

The decode of one layer is the split-KV attention kernel and the combine of
split sequences, run with a schedule built once per decode step and shared
by every layer (topnet.top "Was ist FlashMLA?", "MLA-Metadaten abrufen").
A step here is that per-layer decode over one batch; `value` is its KV-read
bandwidth on the memory-bound variable-length workload (batch 64, 1 query
token, 16 heads, lengths uniform in [1, 8192], bf16 pages): algorithmic KV
bytes / decode time.  The step including the schedule kernel is reported as
`step_with_schedule_ms`.  The compute-bound MTP decode (batch 128, 2 query
tokens, 128 heads, L = 4096, causal) is the metric's bf16-TFLOPS leg
(`roofline_mtp`); the FP8, sparse, prefill and append workloads are under
`secondary`.

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Six physical copies of each page pool (same logical cache, pages shuffled
differently; --replicas) are used in rotation so that consecutive calls do
not hit the 256 MB Infinity Cache.

Timed loops per workload, all replayed from HIP graphs (as a serving loop
runs them) with HIP events on the launch stream around every replay; a
graph holds four rotations of the pool copies (24 calls), so one graph
launch's idle time is shared by 24 calls:
  * decode: per call, the split-KV kernel and the combine (value,
    ms_per_step; mean and p10/p50/p90 over replays);
  * step_with_schedule: per call, the schedule kernel, then the decode;
  * the dominant kernel alone, back to back: its mean launch duration gives
    the roofline's `achieved` (algorithmic bytes or flops per launch over
    it), the figure rocprofv3's kernel trace of the same command reports.
Every graph's output is checked bit for bit against an eager call first.
`roofline.traffic` (measured HBM bytes per launch) is read from the
committed counter summary in profiles/ when it was taken on the kernel
sources as they are now, else null.  `sclk_mhz` is the shader clock sampled
while the MTP graphs run; `hbm_copy_gbs` is the rate of a plain 1 GiB
device copy (read + write bytes over time) and `hbm_read` that of a
plain 1 GiB read (the reference kernel in libmla_bw.so), the streaming
rates simple kernels reach on this part.

    python bench.py --only WORKLOAD --graph-only

times one workload from graph replays only: the run the kernel traces in
profiles/ are taken on.

    python bench.py --pmc-run [membound|mtp|fp8|sparse|...]

runs the workload that the counter summaries are taken on: a plain fp32
copy of known size first (the counters' calibration), then a few eager
calls of the workload.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
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


def _pcts(per_call_ms) -> dict:
    a = np.asarray(per_call_ms, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.median(a)),
            "p90": float(np.percentile(a, 90))}


class Workload:
    """Device-resident inputs (with pool replicas), prepared calls and the
    HIP graphs the timed loops replay."""

    def __init__(self, name: str, replicas: int):
        import torch
        import mla_inputs as gen
        import mla_paged_kv_metadata_amd as m
        self.name = name
        # "<workload>_qk8": the same inputs decoded with the query quantised
        # to e4m3 (qk_fp8, the FP8-MFMA variant)
        self.qk8 = name.endswith("_qk8")
        self.cfg = gen.WORKLOADS[name[:-4] if self.qk8 else name]
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
                             causal=inp.causal, indices=self.indices, out=out, lse=lse, workspace=ws,
                             qk_fp8=self.qk8)
            out, lse, ws = c.out, c.lse, c.workspace
            self.calls.append(c)
        torch.cuda.synchronize()
        self.bytes = algorithmic_bytes(inp)
        self.flops = inp.flops()

    def refresh(self, r):
        import mla_paged_kv_metadata_amd as m
        m.refresh_mla_metadata(self.mds[r], self.seqlens, self.indices)

    def dominant(self, c):
        """Launch the workload's dominant kernel alone: the split-KV kernel."""
        c.partial()

    def eager(self, i, ev=None):
        """One eager step (schedule, then the decode), with HIP events around
        each when ev is given."""
        r = i % len(self.calls)
        c = self.calls[r]
        if ev is not None:
            ev[0].record()
        self.refresh(r)
        if ev is not None:
            ev[1].record()
        c.run()
        if ev is not None:
            ev[2].record()

    def _graph(self, body):
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_ROTATIONS):
                for r, c in enumerate(self.calls):
                    body(r, c)
        return g

    def capture(self):
        """Graphs of GRAPH_ROTATIONS rotations over the pool copies: decode
        calls, schedule + decode calls, and the dominant kernel alone."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(2 * len(self.calls)):
                self.eager(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.per_graph = GRAPH_ROTATIONS * len(self.calls)
        self.g_decode = self._graph(lambda r, c: c.run())
        self.g_step = self._graph(lambda r, c: (self.refresh(r), c.run()))
        self.g_dominant = self._graph(lambda r, c: self.dominant(c))
        torch.cuda.synchronize()

    def check_graphs(self):
        """Each graph's out/lse must equal the eager call's, bit for bit (all
        pool copies hold the same logical cache)."""
        import torch
        c0 = self.calls[0]
        self.eager(0)
        torch.cuda.synchronize()
        ref_o, ref_l = c0.out.clone(), c0.lse.clone()
        for name, g in (("decode", self.g_decode), ("step", self.g_step)):
            c0.out.fill_(0)
            c0.lse.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            if not (torch.equal(c0.out, ref_o) and torch.equal(c0.lse, ref_l)):
                raise RuntimeError(f"{name} graph differs from the eager call")

    def time_graph(self, g, calls: int) -> dict:
        """Replay g until about `calls` calls have run (at least 3 replays),
        with HIP events on the launch stream around every replay; per-call
        ms (mean, p10/p50/p90 over replays)."""
        import torch
        reps = max(3, -(-calls // self.per_graph))
        g.replay()
        g.replay()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(reps):
            g.replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per_call = [evs[i].elapsed_time(evs[i + 1]) / self.per_graph for i in range(reps)]
        out = _pcts(per_call)
        out["calls"] = reps * self.per_graph
        return out

    def time_eager(self, steps: int, warmup: int) -> dict:
        """Eager steps with HIP events between the kernels (the per-kernel
        times include dispatch latency)."""
        import torch
        for i in range(warmup):
            self.eager(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.eager(i, evs[i])
        torch.cuda.synchronize()
        return {
            "metadata_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
            "decode_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
            "step_ms": float(np.mean([e[0].elapsed_time(e[2]) for e in evs])),
        }


def sample_sclk(run, seconds: float):
    """Shader clock (MHz) sampled while `run()` keeps the GPU busy for about
    `seconds`: median and max of the samples, or None if no reader works."""
    import threading
    samples, stop = [], threading.Event()

    def reader():
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]
            while not stop.is_set():
                info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                samples.append(float(info.get("clk", info.get("cur_clk", 0))))
                time.sleep(0.02)
            amdsmi.amdsmi_shut_down()
            return
        except Exception as e:  # noqa: BLE001 - fall back to the command-line tool
            log(f"[bench] amdsmi clock read failed ({e}); trying rocm-smi")
        import re
        import subprocess
        while not stop.is_set():
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                   timeout=10)
                d = json.loads(r.stdout)
                for card in d.values():
                    for k, v in card.items():
                        if "sclk" in k.lower():
                            mm = re.search(r"(\d+)\s*Mhz", str(v), re.I)
                            if mm:
                                samples.append(float(mm.group(1)))
            except Exception:  # noqa: BLE001
                return

    t = threading.Thread(target=reader, daemon=True)
    t.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        run()
    stop.set()
    t.join(timeout=15)
    vals = [v for v in samples if v > 0]
    if not vals:
        return None
    return {"median": float(np.median(vals)), "max": float(max(vals)), "samples": len(vals)}


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


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the oracle's timing line."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, target_s: float, unit: str, threads=None) -> dict:
    """The fp64 oracle on a bounded sample of the same workload: whole
    sequences (all their query rows), taken in order until about target_s of
    CPU work per run; the median of three runs, reported in the metric's
    unit over the sampled sequences (KV-read GB/s, or TFLOP/s)."""
    import oracle
    oracle.build(force=False)
    threads = threads or oracle.max_threads()
    rows_per_b = inp.s_q * inp.h_q
    row_bytes = 1152 if inp.fmt == 0 else 656

    def run(nb):
        sel = np.arange(nb * rows_per_b, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.decode(inp, sel=sel, threads=threads)
        return time.perf_counter() - t0

    # calibrate on the first sequence, then take whole sequences in order
    per_seq = run(1)
    nb = max(1, min(inp.batch, int(target_s / max(per_seq, 1e-4))))
    times = sorted(run(nb) for _ in range(3))
    dt = times[1]
    sub = dataclasses.replace(inp, seqlens=inp.seqlens[:nb], q=inp.q[:nb], block_table=inp.block_table[:nb],
                              indices=None if inp.indices is None else inp.indices[:nb])
    kv = sub.kv_bytes_read()
    flops = sub.flops()
    value = kv / dt / 1e9 if unit == "GB/s" else flops / dt / 1e12
    return {"value": value, "unit": unit, "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {nb} of {inp.batch} sequences, all {rows_per_b} query rows each "
                      f"({kv / 1e6:.1f} MB of KV rows, {flops / 1e9:.2f} GFLOP); median of 3 runs "
                      f"({', '.join(f'{t:.2f}' for t in times)} s)",
            "kv_gbs": kv / dt / 1e9, "tflops": flops / dt / 1e12}


def cpu_tiny_one_thread() -> dict:
    """The oracle on the tiny workload (batch 2, 16 heads, lengths 37 and
    130) with one thread: median of 5 runs."""
    import mla_inputs as gen
    import oracle
    inp = gen.make_inputs(gen.WORKLOADS["tiny"])
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.decode(inp, threads=1)
        ts.append(time.perf_counter() - t0)
    return {"ms": float(np.median(ts)) * 1e3, "cores": 1, "kind": "oracle", "sample": "tiny workload, whole"}


# The dominant kernel of each workload, as rocprofv3 names it, and the
# sources it is built from (the counter summary is valid while they match).
KERNEL_NAMES = {
    "membound": "void mla::narrow::narrow_kernel<0, false>(mla::DecodeParams)",
    "mtp": "mla::wide::offset_kernel(mla::DecodeParams)",
    "fp8": "void mla::wide::wide_kernel<1, false, true>(mla::DecodeParams)",
    "sparse": "void mla::wide::wide_kernel<1, true, true>(mla::DecodeParams)",
    "fp8_qk8": "void mla::wide::wide_kernel<1, false, false>(mla::DecodeParams)",
    "sparse_qk8": "void mla::wide::wide_kernel<1, true, false>(mla::DecodeParams)",
    "sparse_prefill": "void mla::wide::wide_kernel<1, true, true>(mla::DecodeParams)",
    "dense_prefill": "mla::wide::offset_kernel(mla::DecodeParams)",
}
KERNEL_SOURCES = {
    "membound": ["mla_decode_narrow.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "mtp": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "fp8": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "sparse": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "fp8_qk8": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "sparse_qk8": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "sparse_prefill": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
    "dense_prefill": ["mla_decode_wide.hip", "mla_slice.h", "mla_device.h", "mla_internal.h"],
}
# Counter summaries in profiles/: kernel trace + MFMA counters, and HBM
# traffic (FETCH_SIZE / WRITE_SIZE), per workload.
PROFILE_STEM = {
    "membound": "narrow_kernel_membound_b64_h16",
    "mtp": "offset_kernel_mtp_b128_sq2_h128",
    "fp8": "wide_kernel_fp8_b64_h128_L8192",
    "sparse": "wide_kernel_sparse_b32_h128_top2048",
    "fp8_qk8": "wide_kernel_qk8_fp8_b64_h128_L8192",
    "sparse_qk8": "wide_kernel_qk8_sparse_b32_h128_top2048",
    "sparse_prefill": "wide_kernel_sparse_prefill_sq2048_h128_top2048",
    "dense_prefill": "offset_kernel_dense_prefill_sq2048_h128_L8192",
}


def _profile(name: str, kind: str) -> str:
    return os.path.join(ROOT, "profiles", f"{PROFILE_STEM[name]}_{kind}.md")


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
    return _summary_json(_profile(name, "traffic"), "traffic-json", name)


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
    """Kernel trace and MFMA counter figures of the dominant kernel from the
    committed summary, or None."""
    return _summary_json(_profile(name, "kernel_stats"), "mfma-json", name)


def pmc_run(which: str):
    """The run the counter summaries are taken on: a plain copy of known
    size (fp32, 256 Mi elements: 1 GiB read, 1 GiB written: the counters'
    calibration), then six eager calls of the workload's decode."""
    import torch
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
        w.refresh(i % 3)
        w.calls[i % 3].run()
    torch.cuda.synchronize()
    log(f"[bench] pmc run done: 6 calls of {w.cfg.name} ({w.flops} flops, {w.bytes['total']} B per call)")


def run_workload(name: str, replicas: int, steps: int, warmup: int, graph_only: bool = False):
    w = Workload(name, replicas)
    w.capture()
    w.check_graphs()
    t = {"decode": w.time_graph(w.g_decode, steps), "step_with_schedule": w.time_graph(w.g_step, steps),
         "dominant_kernel": w.time_graph(w.g_dominant, steps)}
    if not graph_only:
        t["eager"] = w.time_eager(max(5, steps // 4), warmup)
    return w, t


def copy_rate(reps: int = 10) -> float:
    """HBM rate of a plain device copy (1 GiB read + 1 GiB written per
    copy, torch's copy kernel), GB/s over `reps` back-to-back copies timed
    with HIP events: what a simple streaming kernel reaches on this part."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    rate = 2 * n * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(rate, 1)


def read_rate(reps: int = 10) -> dict:
    """HBM rate of a plain streaming read: the reference kernel of
    libmla_bw.so (16-byte loads, eight in flight per lane, every byte read
    once) over 1 GiB, GB/s over `reps` back-to-back launches timed with HIP
    events, for a few grid sizes; the best is the read rate a simple kernel
    reaches on this part."""
    import ctypes
    import torch
    import mla_paged_kv_metadata_amd as m
    lib = ctypes.CDLL(os.path.join(os.path.dirname(m.__file__), "libmla_bw.so"))
    lib.mla_bw_read.restype = ctypes.c_int
    lib.mla_bw_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    grids = (1024, 2048, 4096, 8192)
    sink = torch.empty(max(grids) * 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rates = {}
    for blocks in grids:
        def launch():
            rc = lib.mla_bw_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
            if rc != 0:
                raise RuntimeError(f"mla_bw_read failed ({rc})")
        for _ in range(2):
            launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        rates[blocks] = round(nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, sink
    torch.cuda.empty_cache()
    best = max(rates, key=rates.get)
    return {"gbs": rates[best], "workgroups": best, "by_workgroups": rates}


def roofline_object(w, t, bound: str) -> dict:
    """Roofline of the dominant kernel: algorithmic bytes (hbm) or flops
    (mfma) per launch over its mean launch duration in the timed graphs."""
    ms = t["dominant_kernel"]["mean"]
    traffic = measured_traffic(w.name)
    if bound == "hbm":
        achieved, peak, unit = w.bytes["total"] / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = w.flops / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    r = {"kernel": KERNEL_NAMES[w.name], "bound": bound, "achieved": round(achieved, 2), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4),
         "traffic": None if traffic is None else int(traffic["bytes_per_launch"]),
         "algorithmic_bytes": w.bytes["total"], "algorithmic_flops": w.flops,
         "kernel_ms": round(ms, 5)}
    if traffic is not None:
        r["traffic_detail"] = {k: traffic[k] for k in ("fetch_bytes", "write_bytes", "fetch_factor",
                                                       "write_factor") if k in traffic}
    mf = measured_mfma(w.name)
    if mf is not None:
        r["rocprof"] = mf
    return r


def summary(w, t) -> dict:
    dec = t["decode"]["mean"] * 1e-3
    return {
        "workload": w.cfg.name,
        "decode_ms": {k: round(v, 5) for k, v in t["decode"].items()},
        "step_with_schedule_ms": {k: round(v, 5) for k, v in t["step_with_schedule"].items()},
        "dominant_kernel": KERNEL_NAMES[w.name],
        "dominant_kernel_ms": {k: round(v, 5) for k, v in t["dominant_kernel"].items()},
        "eager_ms": {k: round(v, 5) for k, v in t["eager"].items()} if "eager" in t else None,
        "tflops": round(w.flops / dec / 1e12, 2),
        "kv_gbs": round(w.bytes["kv"] / dec / 1e9, 1),
        "flops": w.flops,
        "kv_bytes": w.bytes["kv"],
        "num_parts": w.md.num_parts,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--cpu-seconds", type=float, default=5.0, help="CPU work per oracle run (3 runs each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true",
                    help="skip every workload but the memory-bound one")
    ap.add_argument("--only", choices=["membound", "mtp", "fp8", "sparse", "fp8_qk8", "sparse_qk8",
                                       "sparse_prefill", "dense_prefill", "append"], default=None,
                    help="time just this workload (for profiling)")
    ap.add_argument("--graph-only", action="store_true",
                    help="with --only: time the graph replays only (no eager steps), so that a kernel "
                         "trace of the run holds graph-ordered launches apart from the set-up calls")
    ap.add_argument("--pmc-run", nargs="?", const="membound", default=None,
                    choices=["membound", "mtp", "fp8", "sparse", "fp8_qk8", "sparse_qk8", "sparse_prefill",
                             "dense_prefill"],
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
        w, t = run_workload(args.only, args.replicas, args.steps, args.warmup, args.graph_only)
        print(json.dumps(summary(w, t)), flush=True)
        return

    prim, tm = run_workload("membound", args.replicas, args.steps, args.warmup)
    log("[bench] membound timed")
    kv = prim.bytes["kv"]
    dec_ms = tm["decode"]["mean"]
    value = kv / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": "MLA paged decode: KV-read GB/s (h_q=16) and bf16 TFLOPS (h_q=128,s_q=2)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec_ms, 5),
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
            "step": "one layer's decode (split-KV attention + combine) with the step's schedule, "
                    f"replayed from HIP graphs of {GRAPH_ROTATIONS * args.replicas} calls",
        },
        "timing_ms": summary(prim, tm),
        "step_with_schedule_kv_gbs": round(kv / (tm["step_with_schedule"]["mean"] * 1e-3) / 1e9, 1),
        "roofline": roofline_object(prim, tm, "hbm"),
        "hbm_copy_gbs": copy_rate(),
        "hbm_read": read_rate(),
    }
    if not args.only_primary:
        extra = {}
        for key in ("mtp", "fp8", "sparse", "fp8_qk8", "sparse_qk8", "sparse_prefill", "dense_prefill"):
            del prim
            torch.cuda.empty_cache()
            log(f"[bench] timing {key}")
            w, t = run_workload(key, args.replicas, max(24, args.steps // 2), args.warmup)
            extra[key] = summary(w, t)
            extra[key]["roofline"] = roofline_object(w, t, "mfma")
            if key == "mtp":
                result["roofline_mtp"] = extra[key]["roofline"]
                result["sclk_mhz"] = sample_sclk(w.g_decode.replay, 1.5)
                torch.cuda.synchronize()
            prim = w
        log("[bench] timing append")
        extra["append"] = bench_append(max(10, args.steps // 2))
        result["secondary"] = extra
        del prim
    if not args.no_cpu_baseline:
        import mla_inputs as gen
        import oracle
        log("[bench] cpu baseline (oracle)")
        oracle.build(force=False)
        threads = oracle.max_threads()     # every host thread (read before any 1-thread run)
        inp = gen.make_inputs(gen.WORKLOADS["membound"])
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, "GB/s", threads)
        if not args.only_primary:
            for key in ("mtp", "fp8", "sparse"):
                inp = gen.make_inputs(gen.WORKLOADS[key])
                result["secondary"][key]["cpu_baseline"] = cpu_baseline(
                    inp, args.cpu_seconds, "TFLOP/s" if key == "mtp" else "GB/s", threads)
        result["cpu_baseline"]["tiny_one_thread"] = cpu_tiny_one_thread()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

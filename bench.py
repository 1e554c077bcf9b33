#!/usr/bin/env python
"""Benchmark of the DCP LSE merge (dcp_lse_combine) on one MI355X.

A step is one layer-merge: one dcp_lse_combine call over all B tokens of one
synthetic batch (every chunk included), i.e. the whole hot path -- layout
adapter, chunk planner, LSE reduction, weighted accumulation, store.

Timing.  Inputs are resident in HBM before the timed region starts.  Every
timed call reads an input set of its own (up to 32 GiB of sets; past that the
sets are cycled, tens of gigabytes apart): measured, a set read again even
1.27 GB of other inputs later -- five times the 256 MB Infinity Cache -- still
comes back about 9% faster, so no timed call re-reads another's bytes.  After
one untimed call on every set, warm-up calls run on a separate set; then 1 GiB
of unrelated data is read, so every timed input comes from HBM (a cold-cache
figure).  The timed calls are eager launches on one stream, back to back; a
bounded spin kernel queued before the start event keeps the GPU busy while the
host enqueues them (the line reports both times), so the region holds GPU work
only.  The region is bracketed by a barrier and torch.cuda.synchronize() and
measured with HIP events on that stream.  The same calls captured in HIP graphs
of min(60, steps) calls (60: one per MLA layer of a decode step) are reported
beside it: every graph replay adds ~7.5 us of the graph runtime's own start-up
on the GPU, which a 20-call region cannot amortise, while a decode step's graph
pays it once for thousands of kernels.  A hot-cache figure (same buffers every
call) is reported too.

Output: one JSON line (rank 0).  ``value`` is achieved HBM throughput in GB/s
= algorithmic bytes per layer-merge / time per layer-merge, where algorithmic
bytes = sum over (token, local head) of (non-empty shards * 1024 + cp * 4 +
1024 + 4): each non-empty shard's bf16 D-row and every LSE read once, the
merged row and merged LSE written once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per layer-merge + achieved HBM GB/s (% of peak) at B=1..512, 1×MI355X"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
COLD_BYTES = 1 << 30            # unrelated bytes read before the timed region (cache eviction)
DISTINCT_BYTES = 32 << 30       # timed input sets up to this footprint are all distinct
KV_COPIES = 24                  # producer: cache copies in rotation (3.6 GB; a copy is re-read 3.5 GB later)
GRAPH_CALLS = 60                # calls per captured graph (one per MLA layer)
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "dcp_merge_kimi_b128_counters.txt")
MERGE_SRC = os.path.join(ROOT, "context_lse_merge_amd", "csrc", "merge.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=600, help="timed layer-merges (a multiple of 60 above 60)")
    p.add_argument("--warmup", type=int, default=120)
    p.add_argument("--workload", choices=["kimi", "dsv2", "stress", "kimi_f16", "dsv2_f16", "stress_f16", "wide32",
                                          "wide64"],
                   default="kimi")
    p.add_argument("--B", type=int, default=128)
    p.add_argument("--no-sweep", action="store_true", help="skip the B = 1..512 sweep")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-hot", action="store_true", help="skip the hot-cache figure")
    p.add_argument("--no-producer", action="store_true", help="skip the MLA producer (B = 1, 8, 32, 64) leg")
    p.add_argument("--producer-B", type=int, nargs="*", default=[1, 8, 32, 64])
    p.add_argument("--no-fused", action="store_true",
                   help="skip the dcp_mla_decode_merged rows (separate vs fused epilogue) of the producer leg")
    p.add_argument("--calibrate", action="store_true",
                   help="also run a plain 256 MiB elementwise copy kernel (reference for HBM byte counters)")
    return p.parse_args()


def make_case(workload, B):
    import torch
    import synth
    dtype = torch.float16 if workload.endswith("_f16") else torch.bfloat16
    base = workload[:-4] if workload.endswith("_f16") else workload
    if base == "kimi":
        return synth.kimi_merge(B, dtype=dtype)
    if base == "dsv2":
        return synth.dsv2_merge(B, dtype=dtype)
    if base.startswith("wide"):
        return synth.wide_merge(B, int(base[4:]), dtype=dtype)
    return synth.stress_merge(B, dtype=dtype)


def workload_name(case, workload):
    desc = {"kimi": "Kimi-K2.5-like merge, [B,H/cp,cp] base-e LSE",
            "dsv2": "DeepSeek-V2-236B-like merge, FlashMLA [B,H,1] base-2 LSE",
            "stress": "stress merge, 10% empty shards, capacity 128 (ordered chunks)",
            "wide32": "wide merge (16 local heads), [B,H/cp,cp] base-e LSE",
            "wide64": "wide merge (16 local heads), [B,H/cp,cp] base-e LSE"}[workload.replace("_f16", "")]
    return "%s: B=%d H=%d cp=%d H_local=%d D=512 %s" % (desc, case.B, case.H, case.cp, case.h_local,
                                                         "fp16" if workload.endswith("_f16") else "bf16")


def algorithmic_bytes(case):
    """sum over (b, j) of (#non-empty shards * 2D + cp * 4 + 2D + 4)."""
    import torch
    lse = case.lse
    B, H, cp = case.B, case.H, case.cp
    hl = H // cp
    if case.lse_layout == "bh1":
        lse = lse.reshape(B, cp, hl).permute(0, 2, 1)
    nonempty = int(torch.isfinite(lse).sum()) + int((lse == math.inf).sum())
    rows = B * hl
    return nonempty * 1024 + rows * (cp * 4 + 1024 + 4)


class GpuCase:
    """Device copies of one case, replicated into `nsets` input sets."""

    def __init__(self, case, nsets, capacity):
        import torch
        import context_lse_merge_amd as dcp
        self.dcp = dcp
        self.case = case
        dev = torch.device("cuda:0")
        attn0 = case.attn.to(dev)
        lse0 = case.lse.to(dev)
        self.sets = []
        for _ in range(nsets):
            attn = torch.empty_like(attn0)
            attn.copy_(attn0)
            lse = torch.empty_like(lse0)
            lse.copy_(lse0)
            out = torch.empty((case.B, case.h_local, 512), dtype=case.attn.dtype, device=dev)
            out_lse = torch.empty((case.B, case.h_local), dtype=torch.float32, device=dev)
            self.sets.append((attn, lse, out, out_lse))
        self.capacity = capacity
        self.layout = dcp.DCP_LSE_BHC if case.lse_layout == "bhc" else dcp.DCP_LSE_BH1
        self.mode = dcp.DCP_LSE_BASE_E if case.lse_mode == "e" else dcp.DCP_LSE_BASE_2

    def call(self, ws, k, stream):
        attn, lse, out, out_lse = self.sets[k]
        self.dcp.dcp_lse_combine(ws, attn, lse, self.layout, self.mode, out, out_lse, stream=stream)

    def workspace(self, stream, cached=False):
        """A workspace for this case bound to `stream`."""
        import torch
        dtype = self.dcp.DCP_DTYPE_FP16 if self.case.attn.dtype == torch.float16 else self.dcp.DCP_DTYPE_BF16
        ws = self.dcp.dcp_workspace_create(self.capacity, self.case.h_local, self.case.cp, dtype=dtype,
                                           stream=stream)
        if cached:
            self.dcp.dcp_workspace_set_load_policy(ws, self.dcp.DCP_LOAD_CACHED)
        return ws

    def capture(self, set_lists):
        """One HIP graph per list of set indices, calling the sets in that order."""
        import torch
        stream = torch.cuda.Stream()
        dtype = self.dcp.DCP_DTYPE_FP16 if self.case.attn.dtype == torch.float16 else self.dcp.DCP_DTYPE_BF16
        ws = self.dcp.dcp_workspace_create(self.capacity, self.case.h_local, self.case.cp, dtype=dtype,
                                           stream=stream)
        if getattr(self, "cached", False):
            self.dcp.dcp_workspace_set_load_policy(ws, self.dcp.DCP_LOAD_CACHED)
        # one eager pass on the capture stream first
        with torch.cuda.stream(stream):
            for k in range(len(self.sets)):
                self.call(ws, k, stream)
        torch.cuda.synchronize()
        graphs = []
        for ks in set_lists:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for k in ks:
                    self.call(ws, k, stream)
            graphs.append(g)
        torch.cuda.synchronize()
        self.ws = ws
        return graphs


def barrier():
    import torch.distributed as dist
    if dist.is_available() and dist.is_initialized():
        dist.barrier()


_SLEEP_CYCLES_PER_MS = []


def gpu_delay(ms):
    """Queue a spin kernel of about `ms` milliseconds on the current stream (torch's bounded sleep kernel,
    calibrated once with HIP events).  Queued ahead of a start event, it keeps the GPU busy while the host submits
    the graph launches that follow, so the timed region holds GPU work only, not host submission."""
    import torch
    if not _SLEEP_CYCLES_PER_MS:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS.append((1 << 20) / max(e0.elapsed_time(e1), 1e-3))
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS[0]))


_SCRUB = []


def evict_caches():
    """Read 1 GiB that no measurement uses: every cached byte of earlier work (L2, Infinity Cache) is displaced,
    and dirty lines are written back before the timed region, not during it."""
    import torch
    if not _SCRUB:
        _SCRUB.append(torch.ones(COLD_BYTES // 2, dtype=torch.bfloat16, device="cuda:0"))
    torch.sum(_SCRUB[0])


def time_graphs(graphs, replays, evict=False):
    """Replay graphs round-robin from graphs[0], `replays` times; returns elapsed ms, HIP events on the stream the
    replays are launched on, bracketed by a barrier and a synchronize on both sides.  A spin kernel queued before
    the start event covers the host's submission of the replays; with `evict`, 1 GiB of unrelated data is read
    between the spin kernel and the start event."""
    import torch
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    barrier()
    torch.cuda.synchronize()
    gpu_delay(1.0 + 0.05 * replays)
    if evict:
        evict_caches()          # runs right before the start event: the GPU is not idle when timing starts
    start.record(stream)
    for r in range(replays):
        graphs[r % len(graphs)].replay()
    end.record(stream)
    torch.cuda.synchronize()
    barrier()
    return start.elapsed_time(end)


SPIN_MS_PER_CALL = 0.05   # spin time queued per timed call: covers the host's enqueue of one eager call


def time_eager(enqueue, n, evict=False):
    """Run enqueue(i) for i in range(n) -- each one eager launch on the current stream -- as one timed region;
    returns (elapsed ms, host enqueue ms, spin ms).  HIP events on that stream, bracketed by a barrier and a
    synchronize on both sides.  A spin kernel of SPIN_MS_PER_CALL per call queued before the start event keeps
    the GPU busy while the host enqueues the launches, so the region holds GPU work only as long as the host
    enqueue took less than the spin (reported, so a reader can check it); with `evict`, 1 GiB of unrelated data is
    read between the spin kernel and the start event."""
    import torch
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    barrier()
    torch.cuda.synchronize()
    spin_ms = 1.0 + SPIN_MS_PER_CALL * n
    gpu_delay(spin_ms)
    if evict:
        evict_caches()
    start.record(stream)
    t0 = time.perf_counter()
    for i in range(n):
        enqueue(i)
    host_ms = (time.perf_counter() - t0) * 1000.0
    end.record(stream)
    torch.cuda.synchronize()
    barrier()
    return start.elapsed_time(end), host_ms, spin_ms


def warm_up(graph, calls, warmup):
    """Replay a warm-up graph of `calls` calls until at least `warmup` calls ran; returns how many ran."""
    import torch
    if warmup <= 0:
        return 0
    n = math.ceil(warmup / calls)
    for _ in range(n):
        graph.replay()
    torch.cuda.synchronize()
    return n * calls


def plan_sets(per_set, steps, cold):
    """Which input set each timed call reads.  Returns (calls per graph, timed sets, one list of set indices per
    timed graph, the warm-up set).  The timed region replays the graphs in order, round-robin, steps / calls times.
    cold: every timed call reads a set of its own while steps * per_set <= DISTINCT_BYTES, else the calls cycle
    over as many sets as fit in DISTINCT_BYTES (a whole number of graphs, at least one); the warm-up reads the
    next set, which no timed call reads.  hot: set 0 throughout."""
    calls = min(GRAPH_CALLS, steps)
    if steps <= 0 or steps % calls:
        raise SystemExit("--steps must be a positive multiple of %d" % calls)
    if not cold:
        return calls, 1, [[0] * calls], 0
    if steps * per_set <= DISTINCT_BYTES:
        n_sets = steps
    else:
        n_sets = max(1, DISTINCT_BYTES // (per_set * calls)) * calls
    timed = [list(range(g * calls, (g + 1) * calls)) for g in range(n_sets // calls)]
    return calls, n_sets, timed, n_sets


def measure(case, steps, warmup, capacity=None, cold=True, cached=False):
    """Time `steps` layer-merges, each an eager launch (time_eager).

    cold: every timed call reads an input set of its own (plan_sets); after one untimed call on every set, the
    warm-up calls run on a separate set; then 1 GiB of unrelated data is read, so every timed input comes from
    HBM.  hot: every call (warm-up and timed) uses one set.  ``cached``: the workspace's DCP_LOAD_CACHED policy.
    Returns a dict: us per layer-merge, timed input sets, warm-up calls, footprint, first set, host enqueue and
    spin ms."""
    import torch
    per_set = case.attn.numel() * 2 + case.lse.numel() * 4 + case.B * case.h_local * (1024 + 4)
    calls, n_sets, timed, warm_set = plan_sets(per_set, steps, cold)
    order = [k for r in range(steps // calls) for k in timed[r % len(timed)]]
    g = GpuCase(case, max(n_sets, warm_set + 1), capacity or case.B)
    stream = torch.cuda.current_stream()
    ws = g.workspace(stream, cached)
    for k in range(len(g.sets)):
        g.call(ws, k, stream)
    for _ in range(max(0, warmup)):
        g.call(ws, warm_set, stream)
    torch.cuda.synchronize()
    ms, host_ms, spin_ms = time_eager(lambda i: g.call(ws, order[i], stream), steps, evict=cold)
    first = g.sets[0]
    ws.close()
    return {"us": ms * 1000.0 / steps, "sets": n_sets, "warm_calls": max(0, warmup), "footprint": n_sets * per_set,
            "first": first, "reuse_distance_bytes": (n_sets * per_set if steps > n_sets else None),
            "host_ms": host_ms, "spin_ms": spin_ms}


def measure_graphs(case, steps, warmup, capacity=None, cold=True):
    """The same measurement with the calls captured in HIP graphs of min(60, steps) calls, replayed round-robin
    (one replay per 60 calls): every replay adds the graph runtime's own start-up on the GPU, ~7.5 us on MI355X,
    which a 20-call region cannot amortise.  Returns us per layer-merge and the calls per graph."""
    per_set = case.attn.numel() * 2 + case.lse.numel() * 4 + case.B * case.h_local * (1024 + 4)
    calls, n_sets, timed, warm_set = plan_sets(per_set, steps, cold)
    g = GpuCase(case, max(n_sets, warm_set + 1), capacity or case.B)
    w_calls = max(1, min(warmup, calls))
    graphs = g.capture(timed + [[warm_set] * w_calls])
    warm_up(graphs[-1], w_calls, warmup)
    ms = time_graphs(graphs[:-1], steps // calls, evict=cold)
    g.ws.close()
    return {"us": ms * 1000.0 / steps, "calls": calls, "replays": steps // calls}


def launch_floor(steps, warmup):
    """us per launch of a one-element fill kernel (one workgroup) in the same harness as the headline -- eager
    launches on one stream behind a spin kernel -- and, for comparison, in graphs of GRAPH_CALLS launches: the
    fixed cost every layer-merge pays before moving any bytes."""
    import torch
    buf = torch.zeros(1, device="cuda:0")
    for _ in range(max(1, warmup)):
        buf.fill_(1.0)
    torch.cuda.synchronize()
    ms, _, _ = time_eager(lambda i: buf.fill_(1.0), steps)
    eager = ms * 1000.0 / steps
    calls = min(GRAPH_CALLS, steps)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        buf.fill_(1.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(calls):
            buf.fill_(1.0)
    warm_up(g, calls, warmup)
    graph = time_graphs([g], steps // calls) * 1000.0 / steps
    return eager, graph


def copy_ceiling(headline_bytes):
    """Cold device-to-device copies (torch copy_) in the same harness as the headline: eager launches behind a
    spin kernel, after the eviction read.  Returns GB/s (bytes read + written) for 256 MiB copies (over buffers
    cycling through >= 1 GiB; each copy streams more than the Infinity Cache holds), and us per copy that reads and
    writes half of `headline_bytes` each (the same total bytes as one layer-merge; every timed copy has buffers of
    its own, as the merge's timed calls do)."""
    import torch
    res = {}
    n_copies = 5 * GRAPH_CALLS
    for label, nbytes in (("256MiB", 256 << 20), ("headline", headline_bytes // 2)):
        n = max(1, nbytes // 2)
        if n_copies * 2 * n * 2 <= DISTINCT_BYTES:
            sets = n_copies
        else:
            sets = max(2, math.ceil((1 << 30) / (2 * n * 2)))
        src = [torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0) for _ in range(sets)]
        dst = [torch.empty_like(x) for x in src]
        for k in range(min(sets, 4)):
            dst[k].copy_(src[k])
        torch.cuda.synchronize()
        ms, _, _ = time_eager(lambda i: dst[i % sets].copy_(src[i % sets]), n_copies, evict=True)
        us = ms * 1000.0 / n_copies
        res[label] = (us, 2.0 * n * 2 / (us * 1e-6) / 1e9)
        del src, dst
        torch.cuda.empty_cache()
    return {"GBps_256MiB": round(res["256MiB"][1], 1),
            "us_at_headline_bytes": round(res["headline"][0], 3),
            "kernel": "torch copy_ of bf16 buffers, cold, eager launches behind a spin kernel (as the headline); at "
                      "the headline's bytes every timed copy has buffers of its own; GB/s counts bytes read plus "
                      "bytes written"}


def parity_check(case, out, out_lse):
    """The bench's own sanity check of its first input set against the oracle."""
    import numpy as np
    import oracle
    import synth
    olay = oracle.LSE_BHC if case.lse_layout == "bhc" else oracle.LSE_BH1
    omode = oracle.BASE_E if case.lse_mode == "e" else oracle.BASE_2
    r, rL, A = oracle.merge(synth.bits16(case.attn), case.lse.contiguous().numpy(), case.cp, olay, omode,
                            dtype=synth.payload_name(case.attn))
    g = out.float().cpu().double().numpy()
    if synth.payload_name(case.attn) == "f16":
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -14))) - 10)
    else:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
    ok = bool(np.all(np.abs(g - r) <= 2 * ulp + 2.0 ** -16 * A))
    gL = out_lse.cpu().double().numpy()
    fin = np.isfinite(rL)
    ok = ok and bool(np.all(np.abs(gL[fin] - rL[fin]) <= 1e-5 * np.maximum(np.abs(rL[fin]), 1)))
    return ok


def cpu_baseline(case, seconds):
    """The fp64 oracle, as it stands, on the same workload: whole layer-merges
    repeated for about `seconds` (at least 2), all host cores it is allowed."""
    import oracle
    import synth
    bits = synth.bits16(case.attn)
    dt = synth.payload_name(case.attn)
    lse = case.lse.contiguous().numpy()
    olay = oracle.LSE_BHC if case.lse_layout == "bhc" else oracle.LSE_BH1
    omode = oracle.BASE_E if case.lse_mode == "e" else oracle.BASE_2
    threads = len(os.sched_getaffinity(0))
    oracle.merge(bits, lse, case.cp, olay, omode, threads=threads, dtype=dt)          # warm-up
    times = []
    t_end = time.perf_counter() + seconds
    while len(times) < 2 or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        oracle.merge(bits, lse, case.cp, olay, omode, threads=threads, dtype=dt)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    # One thread, for about a third of the budget (at least 2 runs).
    t1 = []
    t_end = time.perf_counter() + seconds / 3
    while len(t1) < 2 or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        oracle.merge(bits, lse, case.cp, olay, omode, threads=1, dtype=dt)
        t1.append(time.perf_counter() - t0)
    t1.sort()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return med * 1e6, threads, len(times), model, t1[len(t1) // 2] * 1e6, len(t1)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16, published
MFMA_FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16, published


def producer_flops(B, hq, T):
    """q.k over 576 columns and p.v over 512, per query row per key."""
    return 2.0 * B * hq * T * (576 + 512)


def measure_producer(B, kv_copies, reps=8, seq_lens=None, replays=5):
    """dcp_mla_partial_decode (+ the merge of its output) on the full-size MLA
    decode workload: q [B,128,576], one 131072 x 576 cache, 4 shards.  The cache
    is rotated over `kv_copies` device copies (KV_COPIES: a copy is read again
    only after 3.5 GB of other copies) so every call reads it from HBM.  With
    `seq_lens` (int32 [B] on the GPU) the variable-length entry point runs
    instead: every token up to its own length, interleaved ownership, over the
    shared cache (kv_sb = 0) or, when the copies are [B, T, 576], over its own
    cache.  q, the cache and the outputs take the cache's dtype.  Both steps are
    timed by batch_call_us in batches of `reps` eager calls: the producer's
    batches each over their own cache copies, in turn, and batches of `reps`
    merges of its output.
    Returns (producer us, merge us) per call, medians over the replays."""
    import torch
    import context_lse_merge_amd as dcp
    import synth
    dev = torch.device("cuda:0")
    hq, cp, T = 128, 4, kv_copies[0].shape[-2]
    dtype = kv_copies[0].dtype
    q = synth.normal_16((B, hq, 576), synth.gen(3000 + B), dtype).to(dev)
    o = torch.empty((B, cp * hq, 512), dtype=dtype, device=dev)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=dev)
    out = torch.empty((B, hq, 512), dtype=dtype, device=dev)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    if seq_lens is None:
        nbytes = dcp.dcp_mla_partial_decode_scratch_size(B, hq, T, cp)
    else:
        nbytes = dcp.dcp_mla_partial_decode_varlen_scratch_size(B, hq, T, cp)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    stream = torch.cuda.Stream()
    ws = dcp.dcp_workspace_create(B, hq, cp, dtype=dcp.DCP_DTYPE_FP16 if dtype == torch.float16 else dcp.DCP_DTYPE_BF16,
                                  stream=stream)
    dcp.dcp_workspace_set_load_policy(ws, dcp.DCP_LOAD_CACHED)   # the partials were just written

    def produce(kv):
        if seq_lens is None:
            dcp.dcp_mla_partial_decode(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, scratch)
        else:
            dcp.dcp_mla_partial_decode_varlen(q, kv, seq_lens, T, dcp.DCP_KV_INTERLEAVED, cp, synth.MLA_SCALE,
                                              dcp.DCP_LSE_BASE_E, o, l, scratch)

    def merge():
        dcp.dcp_lse_combine(ws, o, l, dcp.DCP_LSE_BH1, dcp.DCP_LSE_BASE_E, out, out_lse)

    with torch.cuda.stream(stream):
        for k in range(2):
            produce(kv_copies[k % len(kv_copies)])
            merge()
        torch.cuda.synchronize()
        n_batches = max(1, len(kv_copies) // reps)

        def produce_batch(i):
            for r in range(reps):
                produce(kv_copies[(i * reps + r) % len(kv_copies)])

        def merge_batch(i):
            for _ in range(reps):
                merge()

        prod = batch_call_us(produce_batch, n_batches, reps, replays)
        mrg = batch_call_us(merge_batch, 1, reps, replays)
    ws.close()
    return prod, mrg


PRODUCER_SPIN_MS_PER_CALL = 0.1   # covers the host's enqueue of one producer call (its launches and checks)


def batch_call_us(run_batch, n_batches, reps, replays):
    """us per call of batches of `reps` eager calls on the current stream (run_batch(i) enqueues batch
    i % n_batches): warmed up for about 50 ms of this work (the first ~20 ms of sustained load run measurably
    slower), then at least `replays` batches and at least 20 ms, HIP events around every batch, a spin kernel
    ahead of each start event covering the host's enqueue; the median batch / reps."""
    import torch
    spin = 0.2 + PRODUCER_SPIN_MS_PER_CALL * reps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_delay(spin)
    e0.record()
    run_batch(0)
    e1.record()
    torch.cuda.synchronize()
    once_ms = max(e0.elapsed_time(e1), 1e-3)
    for i in range(int(math.ceil(50.0 / once_ms))):
        run_batch(i % n_batches)
    torch.cuda.synchronize()
    ts = []
    for i in range(max(replays, int(math.ceil(20.0 / once_ms)))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gpu_delay(spin)
        e0.record()
        run_batch(i % n_batches)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[len(ts) // 2] * 1000.0 / reps


def measure_merged(B, kv_copies, fuse, reps=8, replays=5):
    """dcp_mla_decode_merged (the producer's partials and their shard merge in one call) on the full-size MLA
    decode workload, timed as measure_producer times the producer: batches of `reps` eager calls over the rotated
    cache copies (batch_call_us)."""
    import torch
    import context_lse_merge_amd as dcp
    import synth
    dev = torch.device("cuda:0")
    hq, cp, T = 128, 4, kv_copies[0].shape[-2]
    dtype = kv_copies[0].dtype
    q = synth.normal_16((B, hq, 576), synth.gen(3000 + B), dtype).to(dev)
    o = torch.empty((B, cp * hq, 512), dtype=dtype, device=dev)
    l = torch.empty((B, cp * hq), dtype=torch.float32, device=dev)
    out = torch.empty((B, hq, 512), dtype=dtype, device=dev)
    out_lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
    scratch = torch.zeros(dcp.dcp_mla_decode_merged_scratch_size(B, hq, T, cp), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def call(kv):
        dcp.dcp_mla_decode_merged(q, kv, cp, synth.MLA_SCALE, dcp.DCP_LSE_BASE_E, o, l, out, out_lse, fuse=fuse,
                                  scratch=scratch, stream=stream)

    with torch.cuda.stream(stream):
        for k in range(2):
            call(kv_copies[k % len(kv_copies)])
        torch.cuda.synchronize()

        def batch(i):
            for r in range(reps):
                call(kv_copies[(i * reps + r) % len(kv_copies)])

        us = batch_call_us(batch, max(1, len(kv_copies) // reps), reps, replays)
    return us


def fused_rows(Bs, copies):
    """N1: the producer with the split reduction and the shard merge in its epilogue (one launch), and with the two
    reductions in one launch after the decode, against the same work as separate launches, at each B."""
    import context_lse_merge_amd as dcp
    rows = []
    for B in Bs:
        r = {"B": B}
        for name, fuse in (("separate_us", dcp.DCP_FUSE_NONE), ("fused_us", dcp.DCP_FUSE_EPILOGUE),
                           ("reductions_us", dcp.DCP_FUSE_REDUCTIONS), ("auto_us", dcp.DCP_FUSE_AUTO)):
            r[name] = round(measure_merged(B, copies, fuse), 1)
        rows.append(r)
        print("[bench] producer + shard merge B=%d: separate launches %.1f us, fused epilogue %.1f us, "
              "combined reductions %.1f us, auto %.1f us"
              % (B, r["separate_us"], r["fused_us"], r["reductions_us"], r["auto_us"]), file=sys.stderr, flush=True)
    return rows


def producer_leg(Bs, with_fused=True):
    import torch
    import synth
    _, kv = synth.mla_decode(1)
    kv_dev = kv.to("cuda:0")
    copies = [kv_dev] + [kv_dev.clone() for _ in range(KV_COPIES - 1)]
    rows = []
    for B in Bs:
        us, us_m = measure_producer(B, copies)
        fl = producer_flops(B, 128, kv.shape[0])
        tflops = fl / (us * 1e-6) / 1e12
        kv_gbs = kv.numel() * 2 / (us * 1e-6) / 1e9
        rows.append({"B": B, "producer_us": round(us, 1), "merge_us": round(us_m, 3),
                     "TFLOPs": round(tflops, 1), "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "kv_GBps": round(kv_gbs, 1), "flop": fl})
        print("[bench] producer B=%d: %.1f us (%.1f TFLOP/s, %.1f%% of bf16 peak), merge %.2f us"
              % (B, us, tflops, 100 * tflops / MFMA_BF16_PEAK_TFLOPS, us_m), file=sys.stderr, flush=True)
    fused = fused_rows(Bs, copies) if with_fused else []
    # the other payload type and the variable-length entry point, at B = 64
    import numpy as np
    seq = np.random.default_rng(64).integers(1, kv.shape[0] + 1, 64).astype(np.int32)
    seq_dev = torch.from_numpy(seq).to("cuda:0")
    us, us_m = measure_producer(64, copies, seq_lens=seq_dev)
    fl = 2.0 * 128 * float(seq.astype(np.int64).sum()) * (576 + 512)
    tflops = fl / (us * 1e-6) / 1e12
    rows.append({"B": 64, "variant": "variable length: lengths U[1, 131072] (sum %d), one shared cache, "
                                     "interleaved ownership" % int(seq.sum()),
                 "producer_us": round(us, 1), "merge_us": round(us_m, 3), "TFLOPs": round(tflops, 1),
                 "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flop": fl})
    print("[bench] producer varlen B=64 (interleaved, random lengths): %.1f us (%.1f TFLOP/s, %.1f%% of bf16 peak)"
          % (us, tflops, 100 * tflops / MFMA_BF16_PEAK_TFLOPS), file=sys.stderr, flush=True)
    # the same lengths over one cache per token (64 x 131072 rows, 9.7 GB: every row from HBM)
    own = torch.empty((64,) + tuple(kv.shape), dtype=torch.bfloat16, device="cuda:0")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(6400)
    for b in range(64):
        own[b].normal_(0.0, 0.5, generator=gen)
    us, us_m = measure_producer(64, [own], seq_lens=seq_dev)
    del own
    tflops = fl / (us * 1e-6) / 1e12
    rows.append({"B": 64, "variant": "variable length: the same lengths, one cache per token (kv_sb = 131072 rows), "
                                     "interleaved ownership",
                 "producer_us": round(us, 1), "merge_us": round(us_m, 3), "TFLOPs": round(tflops, 1),
                 "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flop": fl})
    print("[bench] producer varlen B=64, per-token caches: %.1f us (%.1f TFLOP/s, %.1f%% of bf16 peak)"
          % (us, tflops, 100 * tflops / MFMA_BF16_PEAK_TFLOPS), file=sys.stderr, flush=True)
    del copies
    copies = [kv_dev.to(torch.float16)]
    copies += [copies[0].clone() for _ in range(KV_COPIES - 1)]
    del kv_dev
    us, us_m = measure_producer(64, copies)
    fl = producer_flops(64, 128, kv.shape[0])
    tflops = fl / (us * 1e-6) / 1e12
    rows.append({"B": 64, "variant": "fp16 q, cache and outputs", "producer_us": round(us, 1),
                 "merge_us": round(us_m, 3), "TFLOPs": round(tflops, 1),
                 "mfma_frac": round(tflops / MFMA_FP16_PEAK_TFLOPS, 4), "flop": fl})
    print("[bench] producer fp16 B=64: %.1f us (%.1f TFLOP/s, %.1f%% of fp16 peak), merge %.2f us"
          % (us, tflops, 100 * tflops / MFMA_FP16_PEAK_TFLOPS, us_m), file=sys.stderr, flush=True)
    del copies
    torch.cuda.empty_cache()
    return rows, fused


def producer_oracle_baseline():
    """The fp64 oracle of the producer (per-shard softmax partials) timed on the
    whole B = 1 workload: 128 query rows over the 131072-key cache, 4 shards,
    36.5 GFLOP, all host cores, one run after a one-row warm-up."""
    import numpy as np
    import oracle
    import synth
    q, kv = synth.mla_decode(1)
    qb, kvb = synth.bf16_bits(q), synth.bf16_bits(kv)
    threads = len(os.sched_getaffinity(0))
    oracle.attention_partials(qb, kvb, 4, synth.MLA_SCALE, oracle.BASE_E, rows=np.arange(1), threads=threads)
    t0 = time.perf_counter()
    oracle.attention_partials(qb, kvb, 4, synth.MLA_SCALE, oracle.BASE_E, rows=np.arange(128), threads=threads)
    dt = time.perf_counter() - t0
    fl = producer_flops(1, 128, kv.shape[0])
    print("[bench] producer oracle B=1: %.2f s (%.2f GFLOP/s fp64, %d threads)" % (dt, fl / dt / 1e9, threads),
          file=sys.stderr, flush=True)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "us": round(dt * 1e6, 1),
            "sample": "the whole B = 1 producer workload (128 query rows x 131072 keys, 4 shards; fp64 C oracle, "
                      "OpenMP over rows), one run"}


CALIBRATION_BYTES = 256 << 20


def calibration_copy():
    """A plain elementwise kernel that reads and writes exactly CALIBRATION_BYTES
    each (bf16 negation), launched 5 times: what FETCH_SIZE / WRITE_SIZE read for
    it converts the counters' units into bytes."""
    import torch
    src = torch.ones(CALIBRATION_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def counters_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when that summary is missing or was taken on a different merge.hip."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    kv = {}
    with open(PROFILE_COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    src_hash = hashlib.sha256(open(MERGE_SRC, "rb").read()).hexdigest()
    if kv.get("merge_hip_sha256") != src_hash:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cache_note(m):
    if m["reuse_distance_bytes"] is None:
        reuse = "each timed call reads an input set no other timed call uses"
    else:
        reuse = "the timed calls cycle over %d input sets, so the same bytes come back only after %.1f GB of " \
                "other inputs" % (m["sets"], m["reuse_distance_bytes"] / 1e9)
    return ("cold: %s; after one untimed call on every set, the warm-up ran on a separate set, then 1 GiB of "
            "unrelated data was read before the timed region" % reuse)


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the merge of one rank's shards is the whole path here, and no "
              "multi-GPU exchange is built; run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import context_lse_merge_amd  # noqa: F401  (fails loudly if the HIP library is missing)

    case = make_case(args.workload, args.B)
    capacity = 128 if args.workload.startswith("stress") else case.B
    alg = algorithmic_bytes(case)
    print("[bench] %s: %d algorithmic bytes per layer-merge" % (workload_name(case, args.workload), alg),
          file=sys.stderr, flush=True)
    # the same calls in HIP graphs first, for comparison (the timed eager calls are then the last merges run)
    head_graph = measure_graphs(case, args.steps, args.warmup, capacity=capacity, cold=True)
    head = measure(case, args.steps, args.warmup, capacity=capacity, cold=True)
    us = head["us"]
    ok = parity_check(case, head["first"][2], head["first"][3])
    us_hot = None if args.no_hot else measure(case, args.steps, args.warmup, capacity=capacity, cold=False)["us"]
    us_hot_cached = None if args.no_hot else measure(case, args.steps, args.warmup, capacity=capacity, cold=False,
                                                     cached=True)["us"]
    gbs = alg / (us * 1e-6) / 1e9
    print("[bench] cold %.3f us (%.1f GB/s; host enqueue %.2f ms behind a %.2f ms spin), in HIP graphs %.3f us, "
          "hot %s us, hot with DCP_LOAD_CACHED %s us, parity %s"
          % (us, gbs, head["host_ms"], head["spin_ms"], head_graph["us"], us_hot, us_hot_cached, ok),
          file=sys.stderr, flush=True)

    sweep = []
    if not args.no_sweep:
        for wl, Bs in (("kimi", [1, 8, 16, 32, 64, 128, 256, 512]), ("dsv2", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]),
                       ("kimi_f16", [64, 128, 512]), ("dsv2_f16", [512]),
                       ("stress", [512]), ("wide32", [16, 32, 64]), ("wide64", [8, 16, 32])):
            for B in Bs:
                c = make_case(wl, B)
                cap = 128 if wl.startswith("stress") else B
                m = measure(c, 120, 60, capacity=cap, cold=True)
                u = m["us"]
                a = algorithmic_bytes(c)
                sweep.append({"workload": wl, "B": B, "us": round(u, 3), "GBps": round(a / (u * 1e-6) / 1e9, 1),
                              "frac_of_peak": round(a / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": a,
                              "input_sets": m["sets"], "footprint_MB": round(m["footprint"] / 1e6, 1),
                              "host_enqueue_covered": m["host_ms"] < m["spin_ms"]})
                print("[bench] sweep %s B=%d: %.3f us, %.1f GB/s" % (wl, B, u, sweep[-1]["GBps"]), file=sys.stderr,
                      flush=True)
        # hot inputs (the same buffers every call, as when the partials were just
        # written): the default streaming policy against DCP_LOAD_CACHED
        for B in (128, 512):
            c = make_case("kimi", B)
            a = algorithmic_bytes(c)
            for cached in (False, True):
                m = measure(c, 120, 60, capacity=B, cold=False, cached=cached)
                u = m["us"]
                sweep.append({"workload": "kimi hot " + ("DCP_LOAD_CACHED" if cached else "DCP_LOAD_STREAMING"),
                              "B": B, "us": round(u, 3), "GBps": round(a / (u * 1e-6) / 1e9, 1),
                              "frac_of_peak": round(a / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes": a,
                              "input_sets": 1, "footprint_MB": round(a / 1e6, 1),
                              "host_enqueue_covered": m["host_ms"] < m["spin_ms"]})
                print("[bench] sweep %s B=%d: %.3f us" % (sweep[-1]["workload"], B, u), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cu, threads, reps, model, cu1, reps1 = cpu_baseline(case, args.cpu_seconds)
        cpu = {"value": round(alg / (cu * 1e-6) / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "us_per_layer_merge": round(cu, 1),
               "sample": "%d whole layer-merges of the same workload (fp64 C oracle, OpenMP over rows, %s); "
                         "median" % (reps, model or "host CPU"),
               "one_thread": {"value": round(alg / (cu1 * 1e-6) / 1e9, 3), "unit": "GB/s",
                              "us_per_layer_merge": round(cu1, 1), "sample": "%d whole layer-merges, median" % reps1}}

    producer, fused = ([], []) if args.no_producer else producer_leg(args.producer_B, not args.no_fused)
    producer_cpu = None
    if not args.no_producer and not args.no_cpu_baseline:
        producer_cpu = producer_oracle_baseline()
    if args.calibrate:
        calibration_copy()
    traffic = counters_traffic()
    floor_us, floor_graph_us = launch_floor(args.steps, args.warmup)
    print("[bench] launch floor: a one-element fill kernel takes %.3f us per launch in the same harness (%.3f us in "
          "HIP graphs of %d)" % (floor_us, floor_graph_us, GRAPH_CALLS), file=sys.stderr, flush=True)
    copy = copy_ceiling(alg)
    print("[bench] copy ceiling: torch copy_ moves 256 MiB at %.1f GB/s (read + write); a copy of the headline's "
          "%d bytes takes %.3f us" % (copy["GBps_256MiB"], alg, copy["us_at_headline_bytes"]), file=sys.stderr,
          flush=True)
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_name(case, args.workload), "B": case.B, "H": case.H, "cp": case.cp,
                   "D": 512, "lse_layout": case.lse_layout, "lse_mode": case.lse_mode, "capacity": capacity,
                   "launch": "each timed call an eager launch on one stream, behind a spin kernel that covers "
                             "the host's enqueue (host %.2f ms, spin %.2f ms)" % (head["host_ms"], head["spin_ms"]),
                   "host_enqueue_covered": head["host_ms"] < head["spin_ms"],
                   "input_sets": head["sets"], "footprint_MB": round(head["footprint"] / 1e6, 1),
                   "warmup_calls_run": head["warm_calls"],
                   "cache": cache_note(head)},
        "us_per_layer_merge": round(us, 3),
        "us_per_layer_merge_hip_graphs": {"us": round(head_graph["us"], 3), "graph_calls": head_graph["calls"],
                                          "replays": head_graph["replays"],
                                          "note": "the same cold calls captured in HIP graphs; each replay adds "
                                                  "the graph runtime's start-up on the GPU, which few calls per "
                                                  "replay cannot amortise"},
        "us_per_layer_merge_hot": None if us_hot is None else round(us_hot, 3),
        "us_per_layer_merge_hot_cached_policy": None if us_hot_cached is None else round(us_hot_cached, 3),
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "launch_floor_us": {"us": round(floor_us, 3), "us_hip_graphs": round(floor_graph_us, 3),
                            "kernel": "one-element fill (one workgroup), eager launches behind a spin kernel as the "
                                      "headline (and in graphs of %d launches)" % GRAPH_CALLS},
        "copy_ceiling": copy,
        "parity_vs_oracle": ok,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg // max(1, math.ceil(case.B / capacity))},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "producer": {"workload": "MLA split-KV decode, q [B,128,576] bf16, latent KV cache 131072 x 576 bf16 in "
                                 "4 contiguous shards, scale 1/sqrt(192), then the merge of its partials",
                     "bound": "mfma (B >= 2), hbm (B = 1)", "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                     "timing": "batches of 8 eager calls behind a spin kernel, %d batches over %d cache copies "
                               "in turn (a copy is read again only after %d others), and batches of 8 merges of "
                               "the just-written partials; ~50 ms of warm-up, then timed per batch; median batch / 8"
                               % (KV_COPIES // 8, KV_COPIES, KV_COPIES - 1),
                     "rows": producer, "cpu_baseline": producer_cpu,
                     "merged": {"what": "dcp_mla_decode_merged: the partials and their shard merge in one call; "
                                        "separate = decode + split reduction + shard merge launches (DCP_FUSE_NONE), "
                                        "fused = one launch whose last-arriving workgroups reduce and merge "
                                        "(DCP_FUSE_EPILOGUE), reductions = decode + one launch that reduces the "
                                        "splits and merges each head's shards in LDS (DCP_FUSE_REDUCTIONS), "
                                        "auto = DCP_FUSE_AUTO",
                                "rows": fused}},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

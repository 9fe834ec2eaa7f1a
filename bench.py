#!/usr/bin/env python3
"""Benchmark of the virtual-rank all-reduce on one MI355X.

Default workload: fused all-reduce (sum) of 8 virtual ranks x 512 MiB bf16
(268,435,456 elements per rank, N(0, 0.01^2) with 1% +-100 outliers), all
buffers resident in the GPU's HBM before timing starts.  One step = one call
of vrc_allreduce (chunk partition on the host, one fused launch that reads
every input once and writes every output once).

Prints ONE JSON line.  `value` is algorithmic HBM throughput of the whole
timed region: 2*N*S bytes per step (read N inputs, write N outputs) over the
wall time per step.  `roofline.achieved` uses the average kernel time from
HIP events recorded on the launch stream; `roofline.traffic` is the measured
HBM bytes per launch from the committed rocprofv3 counter summary, reported
only while the kernel sources still hash to the value recorded with it.
`cpu_baseline` times the CPU oracle (single thread) on a bounded slice of the
same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--mode fused|ring|ring_chained|ring_order|hd|hd_order|select]
       python bench.py --suite | --offsets | --ag-sweep | --overlap [--buckets] | --probe-copy
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
CSRC = os.path.join(ROOT, "ring_all_reduce_virtual_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def alg_bytes(mode: str, n: int, size_bytes: int) -> int:
    """Bytes each mode must move per all-reduce.  Fused and ring-order: read
    N inputs and write N outputs.  Ring and ring-chained: N-1 reduce-scatter
    steps read two chunks and write one per rank (3S per step), N-1
    all-gather steps read and write one chunk per rank (2S per step)."""
    mode = selected(mode, n, size_bytes)
    if mode in ("fused", "ring_order", "hd_order"):
        return 2 * n * size_bytes
    return 5 * (n - 1) * size_bytes


def recorded_traffic(workload: str, mode: str):
    """Measured HBM bytes per launch from profiles/<kernel>.<workload>.counters.md,
    if those counters were taken on the current kernel sources."""
    kernel = {"fused": "k_fused_allreduce_phased", "ring": "k_ring_step", "ring_chained": "k_ring_chain_allreduce",
              "ring_order": "k_ring_chain_allreduce", "hd": "k_ring_step",
              "hd_order": "k_fused_allreduce_butterfly"}.get(mode)
    if kernel is None:
        return None
    path = os.path.join(PROFILES, f"{kernel}.{workload}.counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    m_fetch = re.search(r"fetch_bytes_per_launch:\s*([0-9]+)", text)
    m_write = re.search(r"write_bytes_per_launch:\s*([0-9]+)", text)
    if not (m_hash and m_fetch and m_write) or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_fetch.group(1)) + int(m_write.group(1))


def recorded_mixed_stream():
    """The L2-to-fabric latency and stall figures of the headline kernel's
    mixed read/write stream (profiles/mixed_stream.stream_split.counters.md),
    if they were taken on the current kernel sources."""
    path = os.path.join(PROFILES, "mixed_stream.stream_split.counters.md")
    if not os.path.exists(path):
        return None
    vals = dict(re.findall(r"^([a-z_0-9]+):\s*([0-9a-f.]+)\s*$", open(path).read(), re.M))
    if vals.pop("source_sha256_16", None) != kernel_source_hash():
        return None
    return {k: float(v) for k, v in vals.items()}


def time_calls(fn, steps: int, warmup: int, torch):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        starts[k].record(stream)
        fn()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, kms


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, CPUs this process may
    use, and the CPU model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def cpu_baseline(xs, w, mode: str):
    """The oracle as it stands, single-threaded, on the first 3/8 of every
    rank's buffer (inputs copied to the host beforehand, not timed): about
    12 s of CPU work at 8 x 512 MiB."""
    import oracle
    import workloads

    orc = oracle.get()
    sample = max(1, w.count * 3 // 8)
    hx = [workloads.to_numpy(x.reshape(-1)[:sample]) for x in xs]
    algorithm = selected(mode, w.n, w.count * w.esize)
    fn = {"fused": orc.fused_allreduce, "hd": orc.hd_allreduce, "hd_order": orc.hd_allreduce}.get(
        algorithm, orc.ring_allreduce)
    t0 = time.perf_counter()
    fn(hx, w.dtype)
    dt = time.perf_counter() - t0
    gbs = alg_bytes(mode, w.n, sample * w.esize) / dt / 1e9
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"first {sample} of {w.count} elements of each of the {w.n} ranks "
                   f"({mode} oracle, {dt:.2f} s single-threaded; same algorithmic-byte numerator)"),
    }


def selected(mode: str, n: int, size: int, collective: str = "allreduce") -> str:
    """The algorithm VRC_SELECT runs (the rule stated in include/vrc.h)."""
    if mode != "select":
        return mode
    if n & (n - 1) == 0 and size <= (64 << 20):
        return "hd"
    saved = (n - 1) - 2 * (n - 1).bit_length()
    if collective == "all_gather" and n & (n - 1) and saved > 0 and size <= saved * (128 << 10):
        return "tree"
    return "ring"


def tree_slab_copies(n: int) -> int:
    """Slab copies of the binomial-tree all-gather: every receiving rank's own
    slab at the first gather step (ceil(N/2)), slab j once per set bit of j on
    its way to rank 0, and all N slabs to each of the N - 1 other ranks."""
    return (n + 1) // 2 + sum(bin(j).count("1") for j in range(n)) + n * (n - 1)


def suite_bytes(w, mode: str) -> int:
    """Algorithmic bytes per call for a workload's collective and mode."""
    n, size = w.n, w.count * w.esize
    mode = selected(mode, n, size, w.collective)
    if mode == "tree":
        return 2 * tree_slab_copies(n) * size
    fused_like = mode in ("fused", "ring_order", "hd_order")
    if w.collective == "reduce_scatter" and mode == "hd":
        fused_like = True  # the stand-alone halving-doubling reduce-scatter runs as one butterfly launch
    if w.collective == "allreduce":
        return 2 * n * size if fused_like else 5 * (n - 1) * size
    if w.collective == "reduce_scatter":
        return (n + 1) * size if fused_like else 3 * (n - 1) * size
    if mode == "ring_chained":
        return (2 * n - 1) * n * size  # one input read, N-2 relay reads and N writes per input element
    return n * size + n * n * size if fused_like else 2 * n * n * size


def run_suite(steps: int, torch, vrc, workloads) -> int:
    """Every workload (and the fp16 sweep sizes) in every mode.  For
    workloads whose buffers fit in 512 MiB, an untimed 1 GiB device write
    before each timed call evicts the Infinity Cache (the result is labelled
    "effective"); it also keeps the GPU busy while the host enqueues the
    call, so the event interval holds GPU time only.  Larger workloads run
    back to back.  One JSON line per case on stdout."""
    dev = "cuda:0"
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cases = []
    for w in workloads.WORKLOADS.values():
        cases.append(w)
        cases.extend(w.with_count(c) for c in w.sweep)
    for w in cases:
        xs = workloads.make_inputs(w, dev)
        if w.collective == "allreduce":
            outs = [torch.empty_like(x) for x in xs]
        elif w.collective == "reduce_scatter":
            outs = vrc.vrc_reduce_scatter(xs, dim=w.dim)
        else:
            outs = vrc.vrc_all_gather(xs, dim=w.dim)
        torch.cuda.synchronize()
        size = w.count * w.esize
        footprint = {"allreduce": 2 * w.n * size, "reduce_scatter": (w.n + 1) * size,
                     "all_gather": (w.n + w.n * w.n) * size}[w.collective]
        cached = footprint <= (512 << 20)
        for mode in (vrc.MODES if w.collective == "all_gather" else vrc.REDUCE_MODES):
            def call():
                if w.collective == "allreduce":
                    vrc.vrc_allreduce(xs, recv=outs, mode=mode)
                elif w.collective == "reduce_scatter":
                    vrc.vrc_reduce_scatter(xs, recv=outs, dim=w.dim, mode=mode)
                else:
                    vrc.vrc_all_gather(xs, recv=outs, dim=w.dim, mode=mode)
            for _ in range(5):
                call()
            k = min(steps, 20) if w.count * w.esize >= (256 << 20) else steps
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
            for s0, s1 in evs:
                if cached:
                    flush.zero_()
                s0.record()
                call()
                s1.record()
            torch.cuda.synchronize()
            ms = [s0.elapsed_time(s1) for s0, s1 in evs]
            ms.sort()
            # The same call captured in a HIP graph and replayed: the host
            # launch cost of every kernel of the call disappears.
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                call()
            torch.cuda.synchronize()
            gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
            for s0, s1 in gevs:
                if cached:
                    flush.zero_()
                s0.record()
                graph.replay()
                s1.record()
            torch.cuda.synchronize()
            gms = sorted(s0.elapsed_time(s1) for s0, s1 in gevs)
            del graph
            med, p90 = ms[len(ms) // 2], ms[min(len(ms) - 1, int(0.9 * len(ms)))]
            nb = suite_bytes(w, mode)
            rec = {"workload": w.name, "collective": w.collective, "mode": mode, "dtype": w.dtype, "n_ranks": w.n,
                   "elements_per_rank": w.count, "alg_bytes": nb, "calls": k, "us_median": round(med * 1e3, 2),
                   "us_min": round(ms[0] * 1e3, 2), "us_p90": round(p90 * 1e3, 2),
                   "graph_us_median": round(gms[len(gms) // 2] * 1e3, 2),
                   "GB_per_s": round(nb / (med * 1e-3) / 1e9, 1),
                   "pct_of_peak": round(100 * nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                   "footprint_bytes": footprint,
                   "label": "effective (footprint <= 512 MiB, cache flushed before each call)" if cached
                   else "hbm"}
            if mode == "ring_chained":
                # The chained ring issues the step ring's loads and stores, but re-reads each partial
                # right after storing it, from L2: its GB/s counts bytes issued, not HBM bytes.
                rec["note"] = "bytes issued by the kernel; L2 serves the partial re-reads, so this can exceed HBM peak"
            print(json.dumps(rec), flush=True)
            log(f"{w.name:34s} {mode:13s} {rec['us_median']:10.1f} us  (graph {rec['graph_us_median']:10.1f} us)"
                f"  {rec['GB_per_s']:8.1f} GB/s")
        del xs, outs
        torch.cuda.empty_cache()
    return 0


def interleaved_us(torch, calls: dict, steps: int, rounds: int = 4, flush=None) -> dict:
    """Median HIP-event time (us) of each named call, the calls interleaved
    over `rounds` rounds in one process (the same buffers, the same DRAM
    placement for every call of a pair).  With `flush` (a device tensor),
    each timed call follows an untimed write of it."""
    ms = {k: [] for k in calls}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    for _ in range(rounds):
        for name, fn in calls.items():
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(max(1, steps // rounds))]
            for e0, e1 in evs:
                if flush is not None:
                    flush.zero_()
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            ms[name].extend(e0.elapsed_time(e1) for e0, e1 in evs)
    return {k: sorted(v)[len(v) // 2] * 1e3 for k, v in ms.items()}


def offset_views(torch, xs, offsets):
    """Copies of `xs` placed `offsets[r]` elements into fresh buffers."""
    out = []
    for x, off in zip(xs, offsets):
        buf = torch.empty(x.numel() + 64, dtype=x.dtype, device=x.device)
        v = buf[off:off + x.numel()]
        v.copy_(x.reshape(-1))
        out.append(v)
    return out


def run_offsets(steps: int, torch, vrc, workloads) -> int:
    """Operands on other offsets than their destination's 128-byte grid, each
    timed beside its aligned twin in the same process (one JSON line each):

    * the 8 x 512 MiB bf16 all-reduce with rank r's input r elements and its
      output (3r mod 8) elements into fresh buffers, so no two operands share
      an offset, against the aligned buffers, in every mode;
    * a 5-rank bf16 reduce-scatter of about 819 MiB per rank whose chunk bytes
      are odd multiples of 2 (inputs' chunks off the outputs' grid), against a
      count whose chunks are whole 128-byte multiples."""
    dev = "cuda:0"
    w = workloads.WORKLOADS[workloads.HEADLINE]
    xs = workloads.make_inputs(w, dev)
    ys = [torch.empty_like(x) for x in xs]
    mx = offset_views(torch, xs, list(range(w.n)))
    my = offset_views(torch, ys, [3 * r % 8 for r in range(w.n)])
    for mode in vrc.REDUCE_MODES:
        t = interleaved_us(torch, {
            "aligned": lambda: vrc.vrc_allreduce(xs, recv=ys, mode=mode),
            "offset": lambda: vrc.vrc_allreduce(mx, recv=my, mode=mode)}, steps)
        rec = {"offsets": "allreduce_bf16_n8_512mib, rank r input +r, output +3r mod 8 elements", "mode": mode,
               "aligned_us": round(t["aligned"], 1), "offset_us": round(t["offset"], 1),
               "offset_over_aligned": round(t["offset"] / t["aligned"], 4)}
        print(json.dumps(rec), flush=True)
        log(f"offsets AR {mode:13s} aligned {t['aligned']:9.1f} us  offset {t['offset']:9.1f} us "
            f" x{t['offset'] / t['aligned']:.3f}")
    del xs, ys, mx, my
    torch.cuda.empty_cache()
    n = 5
    whole = n * 85878336  # chunk bytes a multiple of 128
    ragged = n * 85878375  # chunk bytes 171,756,750: chunks 1..4 of the inputs off the outputs' grid
    xw = workloads.random_ranks(n, whole, "bf16", seed=61, device=dev, sigma=1e-2)
    xr = workloads.random_ranks(n, ragged, "bf16", seed=62, device=dev, sigma=1e-2)
    yw = vrc.vrc_reduce_scatter(xw)
    yr = vrc.vrc_reduce_scatter(xr)
    for mode in ("ring", "fused", "ring_chained", "ring_order"):
        t = interleaved_us(torch, {
            "aligned": lambda: vrc.vrc_reduce_scatter(xw, recv=yw, mode=mode),
            "offset": lambda: vrc.vrc_reduce_scatter(xr, recv=yr, mode=mode)}, steps)
        # per-element time, so the two counts compare directly
        a_ns, o_ns = t["aligned"] / whole * 1e3, t["offset"] / ragged * 1e3
        rec = {"offsets": f"reduce_scatter bf16 {n} ranks, count {ragged} (ragged chunks) vs {whole}",
               "mode": mode, "aligned_us": round(t["aligned"], 1), "offset_us": round(t["offset"], 1),
               "offset_over_aligned": round(o_ns / a_ns, 4)}
        print(json.dumps(rec), flush=True)
        log(f"offsets RS {mode:13s} aligned {t['aligned']:9.1f} us  ragged {t['offset']:9.1f} us  x{o_ns / a_ns:.3f}")
    return 0


def split_streams(torch, vrc, xs, outs, collective: str, steps: int, flush=None, dim: int = 0) -> dict:
    """One collective beside the same bytes moved one direction at a time:
    the inputs read by the runtime's reduction (torch.sum), the outputs
    written by its fill kernel, and (all-reduce) each input copied into its
    output by the runtime's device copy.  Times are medians of interleaved
    HIP-event intervals on the same buffers."""
    read_bytes = sum(x.numel() * x.element_size() for x in xs)
    write_bytes = sum(y.numel() * y.element_size() for y in outs)

    def collective_call():
        if collective == "allreduce":
            vrc.vrc_allreduce(xs, recv=outs, mode="fused")
        else:
            vrc.vrc_all_gather(xs, recv=outs, dim=dim, mode="fused")

    def read_only():
        for x in xs:
            x.sum(dtype=torch.float32)

    def write_only():
        for y in outs:
            y.fill_(1)

    calls = {"collective": collective_call, "read_only": read_only, "write_only": write_only}
    if collective == "allreduce":
        calls["copy"] = lambda: [y.copy_(x) for x, y in zip(xs, outs)]
    t = interleaved_us(torch, calls, steps, flush=flush)
    rec = {"read_bytes": read_bytes, "write_bytes": write_bytes,
           "collective_us": round(t["collective"], 2), "read_only_us": round(t["read_only"], 2),
           "write_only_us": round(t["write_only"], 2),
           "read_only_GB_per_s": round(read_bytes / t["read_only"] / 1e3, 1),
           "write_only_GB_per_s": round(write_bytes / t["write_only"] / 1e3, 1),
           "collective_GB_per_s": round((read_bytes + write_bytes) / t["collective"] / 1e3, 1),
           "serialized_us": round(t["read_only"] + t["write_only"], 2),
           "collective_over_serialized": round(t["collective"] / (t["read_only"] + t["write_only"]), 4)}
    if "copy" in t:
        rec["copy_us"] = round(t["copy"], 2)
        rec["copy_GB_per_s"] = round((read_bytes + write_bytes) / t["copy"] / 1e3, 1)
    return rec


def run_stream_split(steps: int, torch, vrc, workloads) -> int:
    """The headline all-reduce (8 x 512 MiB bf16) and the 8-rank fp16 heads
    all-gather, each beside read-only, write-only (and copy) passes over the
    same bytes (split_streams); the all-gather's calls each follow a 1 GiB
    cache flush, as in the suite.  One JSON line per workload; run under
    rocprofv3 --pmc for the per-kernel counters."""
    dev = "cuda:0"
    w = workloads.WORKLOADS[workloads.HEADLINE]
    xs = workloads.make_inputs(w, dev)
    ys = [torch.empty_like(x) for x in xs]
    rec = split_streams(torch, vrc, xs, ys, "allreduce", steps)
    print(json.dumps({"stream_split": w.name, **rec}), flush=True)
    log(f"stream split {w.name}: {rec}")
    del xs, ys
    torch.cuda.empty_cache()
    w = workloads.WORKLOADS["all_gather_fp16_n8_heads"]
    xs = workloads.make_inputs(w, dev)
    outs = vrc.vrc_all_gather(xs, dim=w.dim)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    rec = split_streams(torch, vrc, xs, outs, "all_gather", steps, flush=flush, dim=w.dim)
    print(json.dumps({"stream_split": w.name, **rec}), flush=True)
    log(f"stream split {w.name}: {rec}")
    return 0


def run_ag_sweep(steps: int, torch, vrc, workloads) -> int:
    """The all-gather algorithms side by side: ring relay, recursive doubling
    (halving-doubling's all-gather, powers of two only), binomial tree and the
    fused broadcast, for several rank counts and per-rank sizes (fp16, flat),
    interleaved in one process; a 1 GiB write before each call evicts the
    Infinity Cache for calls whose buffers fit in it.  One JSON line per
    (ranks, size)."""
    dev = "cuda:0"
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    for n in (4, 6, 8, 10, 12, 14, 16):
        for per_rank in (4 << 10, 64 << 10, 256 << 10, 512 << 10, 1 << 20, 8 << 20, 32 << 20, 128 << 20):
            if n * n * per_rank > (8 << 30):
                continue
            count = per_rank // 2
            xs = workloads.random_ranks(n, count, "fp16", seed=90 + n, device=dev)
            ys = vrc.vrc_all_gather(xs)
            modes = ["ring", "tree", "fused", "select"] + (["hd"] if n & (n - 1) == 0 else [])
            cached = (n + n * n) * per_rank <= (512 << 20)
            ms = {m: [] for m in modes}
            for m in modes:
                vrc.vrc_all_gather(xs, recv=ys, mode=m)
            torch.cuda.synchronize()
            for _ in range(4):
                for m in modes:
                    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(max(1, steps // 4))]
                    for e0, e1 in evs:
                        if cached:
                            flush.zero_()
                        e0.record()
                        vrc.vrc_all_gather(xs, recv=ys, mode=m)
                        e1.record()
                    torch.cuda.synchronize()
                    ms[m].extend(e0.elapsed_time(e1) for e0, e1 in evs)
            us = {m: round(sorted(v)[len(v) // 2] * 1e3, 2) for m, v in ms.items()}
            rec = {"ag_sweep": {"n_ranks": n, "bytes_per_rank": per_rank, "us_median": us,
                                "label": "effective" if cached else "hbm"}}
            print(json.dumps(rec), flush=True)
            log(f"all-gather n={n:2d} {per_rank >> 10:7d} KiB/rank: " +
                "  ".join(f"{m} {t:9.1f}" for m, t in us.items()))
            del xs, ys
            torch.cuda.empty_cache()
    return 0


def run_overlap(steps: int, mode: str, torch, vrc, workloads) -> int:
    """Overlap of the all-reduce with compute on two streams (the pages'
    compute/communication overlap: the collective runs on its own stream,
    started and joined through events).  A bf16 8192^3 matmul stream stands
    in for backward compute; the all-reduce is the headline workload.  Times
    each alone and both together, each the median of `steps` repetitions.
    One JSON line."""
    dev = "cuda:0"
    w = workloads.WORKLOADS[workloads.HEADLINE]
    xs = workloads.make_inputs(w, dev)
    ys = [torch.empty_like(x) for x in xs]
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(8192, 8192, generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
    s_comp, s_comm = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()

    def timed(launch):
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            s_comp.wait_event(e0)
            s_comm.wait_event(e0)
            launch()
            cur.wait_event(s_comp.record_event())
            cur.wait_event(s_comm.record_event())
            e1.record(cur)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        return ms[len(ms) // 2]

    def gemms(k):
        with torch.cuda.stream(s_comp):
            for _ in range(k):
                torch.matmul(a, b, out=c)

    def allreduce():
        vrc.vrc_allreduce(xs, recv=ys, mode=mode, stream=s_comm)

    gemms(3)
    allreduce()
    torch.cuda.synchronize()
    t_one = timed(lambda: gemms(1))
    t_ar = timed(allreduce)
    k = max(1, round(t_ar / t_one))  # about as much compute as communication
    t_gemm = timed(lambda: gemms(k))
    t_both = timed(lambda: (gemms(k), allreduce()))
    hidden = (t_gemm + t_ar - t_both) / min(t_gemm, t_ar)
    flops = 2 * 8192**3 * k
    out = {"overlap": {"mode": mode, "gemms": k, "gemm_shape": [8192, 8192, 8192], "gemm_ms": round(t_gemm, 4),
                       "gemm_TFLOP_per_s": round(flops / (t_gemm * 1e-3) / 1e12, 1),
                       "allreduce_ms": round(t_ar, 4), "both_ms": round(t_both, 4),
                       "serial_ms": round(t_gemm + t_ar, 4), "fraction_of_shorter_hidden": round(hidden, 3),
                       "workload": w.name}}
    log(f"overlap: {out['overlap']}")
    print(json.dumps(out), flush=True)
    return 0


def run_overlap_buckets(steps: int, mode: str, torch, vrc, workloads, only=None) -> int:
    """The pages' recipe for hiding the all-reduce behind the computation that
    produces its input (www.bjdmk.com.cn/news/5966809/, sections 4.2-4.3): the
    compute stream writes the gradients bucket by bucket and records an event
    per bucket; the communication stream waits on each event and all-reduces
    that bucket (vrc_allreduce_bucketed).  The producer of bucket k is one GEMM
    per rank, [rows_k, K] x [K, 4096] in bf16, written straight into that
    rank's bucket: K = 512 makes all buckets together take about as long as
    the all-reduce (the GEMMs write as many bytes as the all-reduce reads),
    K = 4096 makes them compute-bound, like a weight gradient summed over many
    tokens.  For each bucket size: the GEMMs alone, the bucketed all-reduce
    alone (no waits), and both; `exposed_ms` = both - GEMMs alone is the
    communication the overlap failed to hide.  Totals: the 8 x 512 MiB bf16
    gradients (buckets from 1 MiB per rank), and 8 x 16 MiB (buckets from
    64 KiB, K = 512).  One JSON line per case."""
    dev = "cuda:0"
    n, cols = 8, 4096
    g = torch.Generator(device=dev).manual_seed(11)
    s_comp, s_comm = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()

    def timed(launch, reps):
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            s_comp.wait_event(e0)
            s_comm.wait_event(e0)
            launch()
            cur.wait_event(s_comp.record_event())
            cur.wait_event(s_comm.record_event())
            e1.record(cur)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        return ms[len(ms) // 2]

    series = ((512 << 20, 512, (1 << 20, 4 << 20, 16 << 20, 64 << 20, 256 << 20, 512 << 20)),
              (512 << 20, 4096, (4 << 20, 16 << 20, 64 << 20, 128 << 20, 256 << 20, 512 << 20)),
              (16 << 20, 512, (64 << 10, 256 << 10, 1 << 20, 4 << 20, 16 << 20)))
    if only is not None:  # one case: (K, bucket MiB per rank) on the 8 x 512 MiB gradients
        series = ((512 << 20, only[0], (only[1] << 20,)),)
    for per_rank, k_dim, buckets in series:
        count = per_rank // 2
        rows = count // cols
        grads = [torch.empty(rows, cols, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        outs = [torch.empty_like(x) for x in grads]
        a = torch.randn(rows, k_dim, generator=g, device=dev).to(torch.bfloat16)
        wt = torch.randn(k_dim, cols, generator=g, device=dev).to(torch.bfloat16)
        flat_g = [x.view(-1) for x in grads]
        flat_o = [x.view(-1) for x in outs]
        for bucket_bytes in buckets:
            b_rows = bucket_bytes // 2 // cols
            nb = rows // b_rows
            events = [torch.cuda.Event() for _ in range(nb)]

            def produce(record):
                with torch.cuda.stream(s_comp):
                    for k in range(nb):
                        for x in grads:
                            torch.matmul(a[k * b_rows:(k + 1) * b_rows], wt, out=x[k * b_rows:(k + 1) * b_rows])
                        if record:
                            events[k].record(s_comp)

            def reduce(ready):
                vrc.vrc_allreduce_bucketed(flat_g, recv=flat_o, bucket=b_rows * cols, mode=mode,
                                           ready=events if ready else None, stream=s_comm)

            produce(True)
            reduce(True)
            torch.cuda.synchronize()
            reps = max(3, min(steps, 10))
            t_comp = timed(lambda: produce(False), reps)
            t_ar = timed(lambda: reduce(False), reps)
            t_both = timed(lambda: (produce(True), reduce(True)), reps)
            rec = {"overlap_buckets": {
                "mode": mode, "n_ranks": n, "bytes_per_rank": per_rank, "bucket_bytes_per_rank": bucket_bytes,
                "buckets": nb, "gemm": [b_rows, k_dim, cols], "compute_ms": round(t_comp, 4),
                "allreduce_ms": round(t_ar, 4), "both_ms": round(t_both, 4), "serial_ms": round(t_comp + t_ar, 4),
                "exposed_ms": round(t_both - t_comp, 4),
                "hidden_fraction_of_allreduce": round((t_comp + t_ar - t_both) / t_ar, 3)}}
            print(json.dumps(rec), flush=True)
            log(f"K={k_dim:4d} {per_rank >> 20:4d} MiB/rank in {bucket_bytes >> 10:7d} KiB: compute {t_comp:8.3f} ms  "
                f"all-reduce {t_ar:8.3f}  both {t_both:8.3f}  exposed {t_both - t_comp:8.3f} ms")
        del grads, outs, a, wt, flat_g, flat_o
        torch.cuda.empty_cache()
    return 0


# The measured rows: (workload[@count], mode), every collective of every
# workload in its fused and step-ring forms, plus the headline's other modes.
PROFILE_ROWS = (
    ("allreduce_int32_n4_4099", "fused"), ("allreduce_int32_n4_4099", "ring"),
    ("allreduce_fp32_n8_16mib", "fused"), ("allreduce_fp32_n8_16mib", "ring"),
    ("allreduce_fp16_n8_128mib@524288", "fused"), ("allreduce_fp16_n8_128mib@524288", "ring"),
    ("allreduce_fp16_n8_128mib@8388608", "fused"), ("allreduce_fp16_n8_128mib@8388608", "ring"),
    ("allreduce_fp16_n8_128mib", "fused"), ("allreduce_fp16_n8_128mib", "ring"),
    ("allreduce_bf16_n8_512mib", "fused"), ("allreduce_bf16_n8_512mib", "ring"),
    ("allreduce_bf16_n8_512mib", "ring_chained"), ("allreduce_bf16_n8_512mib", "ring_order"),
    ("allreduce_bf16_n8_512mib", "hd"), ("allreduce_bf16_n8_512mib", "hd_order"),
    ("all_gather_fp16_n8_heads", "fused"), ("all_gather_fp16_n8_heads", "ring"),
    ("reduce_scatter_fp16_n8_act", "fused"), ("reduce_scatter_fp16_n8_act", "ring"),
)
# The headline all-reduce with every operand on its own offset (rank r's input r elements and its output
# 3r mod 8 elements into fresh buffers, as in --offsets), in every all-reduce mode: the single-launch modes
# run their realigned kernels here.
OFFSET_SUFFIX = "+offsets"
PROFILE_OFFSET_ROWS = tuple(("allreduce_bf16_n8_512mib" + OFFSET_SUFFIX, m)
                            for m in ("fused", "hd_order", "ring_order", "ring_chained", "ring"))


def run_profile_case(case: str, steps: int, torch, vrc, workloads) -> int:
    """`steps` calls of each case, each call after an untimed 1 GiB write
    (the suite's cache flush), for rocprofv3 passes: per-dispatch counters
    then belong to the case whose line was printed last before them, and the
    flush's fill kernel separates the calls.  `case` is WORKLOAD[@COUNT]:MODE
    (COUNT overrides the per-rank element count, as the sweep sizes of a
    workload; a "+offsets" suffix on an all-reduce workload puts every
    operand on its own offset, as --offsets does), several joined by commas,
    "rows" for PROFILE_ROWS or "offsets" for PROFILE_OFFSET_ROWS.  One JSON
    line per case, printed (and flushed) before its calls."""
    dev = "cuda:0"
    cases = {"rows": PROFILE_ROWS, "offsets": PROFILE_OFFSET_ROWS}.get(case)
    cases = cases or tuple(tuple(c.split(":")) for c in case.split(","))
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    loaded = xs = outs = None
    for idx, (name, mode) in enumerate(cases):
        shifted = name.endswith(OFFSET_SUFFIX)
        plain = name[:len(name) - len(OFFSET_SUFFIX)] if shifted else name
        base, count = (plain.split("@") + [None])[:2]
        w = workloads.WORKLOADS[base]
        if count is not None:
            w = w.with_count(int(count))
        if shifted and w.collective != "allreduce":
            raise ValueError(f"{name}: operand offsets are profiled for all-reduce workloads only")
        if loaded is None or loaded[0] != name:
            loaded = xs = outs = call = None  # drop the previous workload's buffers before allocating the next
            torch.cuda.empty_cache()
            xs = workloads.make_inputs(w, dev)
            if w.collective == "allreduce":
                outs = [torch.empty_like(x) for x in xs]
                if shifted:
                    xs = offset_views(torch, xs, list(range(w.n)))
                    outs = offset_views(torch, outs, [3 * r % 8 for r in range(w.n)])
            elif w.collective == "reduce_scatter":
                outs = vrc.vrc_reduce_scatter(xs, dim=w.dim)
            else:
                outs = vrc.vrc_all_gather(xs, dim=w.dim)
            loaded = (name, (xs, outs))
        xs, outs = loaded[1]

        def call(w=w, xs=xs, outs=outs, mode=mode):
            if w.collective == "allreduce":
                vrc.vrc_allreduce(xs, recv=outs, mode=mode)
            elif w.collective == "reduce_scatter":
                vrc.vrc_reduce_scatter(xs, recv=outs, dim=w.dim, mode=mode)
            else:
                vrc.vrc_all_gather(xs, recv=outs, dim=w.dim, mode=mode)

        torch.cuda.synchronize()
        print(json.dumps({"profile_case": f"{name}:{mode}", "index": idx, "calls": steps,
                          "collective": w.collective, "n_ranks": w.n, "dtype": w.dtype,
                          "elements_per_rank": w.count, "alg_bytes_per_call": suite_bytes(w, mode)}), flush=True)
        for _ in range(steps):
            flush.zero_()
            call()
        torch.cuda.synchronize()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the 8 x 512 MiB bf16 all-reduce)")
    ap.add_argument("--mode", default="fused",
                    choices=["fused", "ring", "ring_chained", "ring_order", "hd", "hd_order", "select"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the extra ring-mode timing")
    ap.add_argument("--overlap", action="store_true",
                    help="time the all-reduce alone, a matmul stream alone, and both on two streams")
    ap.add_argument("--buckets", action="store_true",
                    help="with --overlap: the bucketed all-reduce behind the GEMMs that produce each bucket, "
                         "swept over bucket sizes")
    ap.add_argument("--bucket-case", default=None,
                    help="with --overlap --buckets: one case only, 'K,MiB' (GEMM depth, bucket MiB per rank)")
    ap.add_argument("--suite", action="store_true",
                    help="measure every workload in every mode (one JSON line each) instead of the headline")
    ap.add_argument("--offsets", action="store_true",
                    help="time operands off their destination's grid beside their aligned twins")
    ap.add_argument("--ag-sweep", action="store_true",
                    help="time the all-gather algorithms (ring, recursive doubling, tree, fused) by size")
    ap.add_argument("--stream-split", action="store_true",
                    help="time the headline all-reduce and the heads all-gather beside read-only, write-only "
                         "and copy passes over the same bytes")
    ap.add_argument("--profile-case", default=None,
                    help="WORKLOAD[@COUNT][+offsets]:MODE[,...], 'rows' or 'offsets' -- run only these "
                         "collectives `--steps` times each (for counter passes)")
    ap.add_argument("--probe-copy", action="store_true",
                    help="only run torch's device copy of 1 GiB (known HBM traffic: 1 GiB read, 1 GiB "
                         "written per launch), for calibrating rocprofv3 byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs N virtual ranks on ONE GPU; --gpus must be 1 "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        return 2

    import torch

    import ring_all_reduce_virtual_amd as vrc
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr, flush=True)
        return 1
    if args.suite:
        return run_suite(args.steps, torch, vrc, workloads)
    if args.offsets:
        return run_offsets(args.steps, torch, vrc, workloads)
    if args.ag_sweep:
        return run_ag_sweep(args.steps, torch, vrc, workloads)
    if args.profile_case:
        return run_profile_case(args.profile_case, args.steps, torch, vrc, workloads)
    if args.stream_split:
        return run_stream_split(args.steps, torch, vrc, workloads)
    if args.overlap and args.buckets:
        only = tuple(int(v) for v in args.bucket_case.split(",")) if args.bucket_case else None
        return run_overlap_buckets(args.steps, args.mode, torch, vrc, workloads, only)
    if args.overlap:
        return run_overlap(args.steps, args.mode, torch, vrc, workloads)
    if args.probe_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes_read_per_launch": 1 << 30, "bytes_written_per_launch": 1 << 30,
                          "launches": args.steps}), flush=True)
        return 0
    w = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    if w.collective != "allreduce":
        print("bench.py: only all-reduce workloads are benchmarked", file=sys.stderr, flush=True)
        return 2
    dev = "cuda:0"
    size = w.count * w.esize
    log(f"workload {w.name}: {w.n} ranks x {size / 2**20:.0f} MiB {w.dtype}, mode {args.mode}")
    xs = workloads.make_inputs(w, dev)
    ys = [torch.empty_like(x) for x in xs]
    torch.cuda.synchronize()
    log("inputs resident in HBM")
    # Fingerprint of the seeded inputs: SHA-256 of each rank's first 16 MiB (the full 4 GiB would take seconds).
    fp_bytes = min(size, 16 << 20)
    fingerprints = [hashlib.sha256(x.reshape(-1).view(torch.uint8)[:fp_bytes].cpu().numpy().tobytes()).hexdigest()[:16]
                    for x in xs]

    def step():
        vrc.vrc_allreduce(xs, recv=ys, mode=args.mode)

    wall, kms = time_calls(step, args.steps, args.warmup, torch)
    nbytes = alg_bytes(args.mode, w.n, size)
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    kavg = sum(kms) / len(kms)
    achieved = nbytes / (kavg * 1e-3) / 1e9
    log(f"{args.steps} steps: {ms_per_step:.4f} ms/step wall, kernel avg {kavg:.4f} ms "
        f"min {min(kms):.4f} ms -> {achieved:.1f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of peak)")

    extra = {"kernel_ms_avg": round(kavg, 5), "kernel_ms_min": round(min(kms), 5),
             "alg_bytes_per_step": nbytes, "kernel_source_sha256_16": kernel_source_hash(),
             "inputs": {"seed": w.seed, "sha256_16_of_first_bytes": fp_bytes, "per_rank": fingerprints}}
    if not args.no_extra:
        for other in vrc.REDUCE_MODES:
            if other == args.mode:
                continue

            def step_other(other=other):
                vrc.vrc_allreduce(xs, recv=ys, mode=other)

            k2 = max(3, min(args.steps, 10))
            wall2, kms2 = time_calls(step_other, k2, 2, torch)
            nb2 = alg_bytes(other, w.n, size)
            extra[f"{other}_mode"] = {
                "steps": k2, "ms_per_step": round(wall2 * 1e3 / k2, 5),
                "GB_per_s": round(nb2 / (wall2 / k2) / 1e9, 2), "alg_bytes_per_step": nb2,
                "launches_per_step": {"ring": 2 * (w.n - 1), "hd": 2 * (w.n.bit_length() - 1)}.get(
                    selected(other, w.n, size), 1),
            }
            if other == "ring_chained":
                extra[f"{other}_mode"]["note"] = "bytes issued; L2 serves the partial re-reads"
            log(f"{other} mode: {extra[f'{other}_mode']}")

        # In place (every rank's output is its input), as a data-parallel gradient all-reduce calls it.
        # It runs on copies, so the timed inputs stay as drawn; each call's sums feed the next call.
        zs = [x.clone() for x in xs]

        def step_in_place():
            vrc.vrc_allreduce(zs, recv=zs, mode=args.mode)

        k4 = max(3, min(args.steps, 10))
        wall4, kms4 = time_calls(step_in_place, k4, 2, torch)
        kavg4 = sum(kms4) / len(kms4)
        extra["in_place"] = {"steps": k4, "ms_per_step": round(wall4 * 1e3 / k4, 5), "kernel_ms_avg": round(kavg4, 5),
                             "GB_per_s": round(nbytes / (kavg4 * 1e-3) / 1e9, 2),
                             "note": "recv = send on copies of the inputs; timing only (the sums compound)"}
        log(f"in place: {extra['in_place']}")
        zs = None
        torch.cuda.empty_cache()

        # The same bytes moved by the runtime's own device copy, on the same buffers in the same process:
        # how close the kernel comes to what this machine's HBM gives a plain N-in/N-out stream.
        def copy_step():
            for x, y in zip(xs, ys):
                y.copy_(x)

        k3 = max(3, min(args.steps, 10))
        wall3, kms3 = time_calls(copy_step, k3, 2, torch)
        copy_gbs = 2 * w.n * size / (sum(kms3) / len(kms3) * 1e-3) / 1e9
        extra["same_box_copy"] = {"what": f"torch copy_ of each rank's input into its output ({w.n} launches, "
                                          f"2*N*S bytes)", "ms_per_step": round(wall3 * 1e3 / k3, 5),
                                  "GB_per_s": round(copy_gbs, 2),
                                  "kernel_over_copy": round(achieved / copy_gbs, 4)}
        log(f"same-box copy: {extra['same_box_copy']}")

        # The mixed stream against one-direction passes over the same bytes (split_streams), with the
        # recorded L2-to-fabric counters: where the remaining gap to the HBM peak comes from.
        split = split_streams(torch, vrc, xs, ys, "allreduce", max(8, min(args.steps, 20)))
        extra["mixed_stream"] = {
            "fused_GB_per_s": split["collective_GB_per_s"], "write_only_GB_per_s": split["write_only_GB_per_s"],
            "copy_GB_per_s": split["copy_GB_per_s"], "write_only_what": "torch fill_ of the 8 outputs",
            "counters": recorded_mixed_stream(),
            "reading": "the kernel reads each phase (0.5-1 GiB) before it writes it, so its reads wait about as "
                       "long as a read-only stream's instead of queueing behind DRAM read/write turnarounds; the rest "
                       "of the gap to the read-then-write bound is the meetings, the turn at each phase boundary, "
                       "the odd XCDs' slower stores (their workgroups hold fewer sums per phase) and fewer reads in "
                       "flight"}
        log(f"mixed stream: {extra['mixed_stream']}")

    # NCCL-style figures for context: algbw = S / t per rank buffer, busbw = algbw * 2(N-1)/N.
    algbw = size / (kavg * 1e-3) / 1e9
    extra["nccl_style"] = {"algbw_GB_per_s": round(algbw, 2),
                           "busbw_GB_per_s": round(algbw * 2 * (w.n - 1) / w.n, 2),
                           "note": "context only; kernel time, S = one rank's buffer"}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a slice of the inputs")
        cpu = cpu_baseline(xs, w, args.mode)
        log(f"cpu baseline {cpu['value']} GB/s")
        extra["cpu_baseline_host"] = host_info()

    out = {
        "metric": "emulated all-reduce HBM GB/s and % of peak, 8 ranks x 512 MB; bit-exact/tol",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "collective": "allreduce", "mode": args.mode, "n_ranks": w.n,
                   "elements_per_rank": w.count, "bytes_per_rank": size, "values": w.note,
                   "parallelism": f"{w.n} virtual ranks in one GPU's HBM"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, args.mode)},
        "cpu_baseline": cpu,
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

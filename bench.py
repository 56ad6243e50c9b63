"""Decode-step benchmark: one paged-attention decode step (decode + split-KV merge) over a
synthetic Llama-8B-shaped batch, on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--schedule S] [--kv F]

Prints ONE JSON line.  value = algorithmic KV bytes per step / wall time per step (GB/s), with
inputs resident in HBM; the timed region is K back-to-back steps, each one prepared-plan call
(decode + merge), bracketed by synchronisation.  Several identical copies of the KV pools are
rotated across steps so that no step finds its KV in the 256 MB last-level (MALL) cache.
graph_us_per_step replays the same steps from a HIP graph.  roofline.achieved divides the same
KV bytes by the decode kernel's own average duration, from HIP events recorded on the launch
stream around every decode launch of a second pass of the same launches.  With the default
arguments the line also carries rows for the other workloads (the mixed batch with window and
sinks, the long-context step, the head-size sweep, an FP8 cache, 512 new tokens per sequence).
cpu_baseline times the fp64 oracle on the host's cores before the GPU is touched.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read GB/s (% of HBM peak) + µs/decode step, bf16 d=128 GQA paged decode"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of one MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCES = ["paged_kv_attention_attn_amd/csrc/pa_decode.hip",
                  "paged_kv_attention_attn_amd/csrc/pa_balanced.hip",
                  "paged_kv_attention_attn_amd/csrc/pa_qk.hpp",
                  "paged_kv_attention_attn_amd/csrc/pa_device.hpp"]


def _code_only(text: str) -> str:
    """C++ source with comments and blank space removed: comment-only edits leave the kernels,
    and so the counters taken on them, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and spacing excluded)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, schedule: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs, if they were taken
    on the current kernel source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    for r in rec.get("records", []):
        if r.get("workload") == workload and r.get("schedule") == schedule:
            return r.get("hbm_bytes_per_launch")
    return None


def attended_pairs(wl) -> int:
    """(query token, key) pairs one query head attends over the batch: token i of q_len new
    tokens sits at position p = L - q_len + i and attends keys max(0, p + 1 - W) .. p (all keys
    up to p when W = 0); p < 0 attends nothing."""
    import numpy as np

    L = wl.seq_lens.astype(np.int64)[:, None]
    p = L - wl.q_len + np.arange(wl.q_len, dtype=np.int64)[None, :]
    n = np.where(p >= 0, p + 1, 0)
    if wl.window > 0:
        n = np.minimum(n, wl.window)
    return int(n.sum())


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The oracle baseline runs in worker processes forked before this process touches the GPU; the
# workload reaches them through this module global (shared copy-on-write by the fork).
_CPU_WL = None
MAX_CPU_WORKERS = 16   # the host share of one GPU on the measurement boxes


def _oracle_step(wl, lo: int, hi: int) -> None:
    """The fp64 oracle over sequences [lo, hi) of the workload (one call of the oracle as it
    stands, on a slice of the batch)."""
    from oracle import ref

    fn = ref.decode_multi if wl.q_len > 1 else ref.decode
    fn(wl.q[lo:hi], wl.k_cache, wl.v_cache, wl.block_table[lo:hi], wl.seq_lens[lo:hi], wl.scale,
       wl.block_size, window=wl.window, sinks=wl.sinks, kv_format=wl.kv_format,
       k_scale=wl.k_scale, v_scale=wl.v_scale)


def _oracle_one_sequence(b: int) -> None:
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        _oracle_step(_CPU_WL, b, b + 1)


def cpu_baseline(wl, min_seconds: float = 8.0) -> dict:
    """The fp64 oracle on this host over the whole step's batch, repeated until at least
    ``min_seconds`` have passed, two ways: on all host cores the process may use (up to 16 worker
    processes, one sequence per task, one BLAS thread each) and on one thread.  The value is
    the all-cores rate.  Must run before the GPU is initialised (the workers are forked)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    global _CPU_WL
    _CPU_WL = wl
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        cores = os.cpu_count() or 1
    cores = max(1, min(MAX_CPU_WORKERS, cores))
    B = wl.num_seqs
    order = sorted(range(B), key=lambda b: -int(wl.seq_lens[b]))   # longest first
    reps_all, dt_all = 0, 0.0
    with mp.get_context("fork").Pool(cores) as pool:
        while dt_all < min_seconds:
            t0 = time.perf_counter()
            pool.map(_oracle_one_sequence, order, chunksize=1)
            dt_all += time.perf_counter() - t0
            reps_all += 1
    reps_one, dt_one = 0, 0.0
    with threadpool_limits(1):
        while dt_one < min_seconds:
            t0 = time.perf_counter()
            _oracle_step(wl, 0, B)
            dt_one += time.perf_counter() - t0
            reps_one += 1
    _CPU_WL = None
    gb = wl.kv_bytes() / 1e9
    return {"value": round(gb * reps_all / dt_all, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds_per_step": round(dt_all / reps_all, 4),
            "repeats": reps_all, "cpu_model": _cpu_model(),
            "one_thread": {"value": round(gb * reps_one / dt_one, 4), "unit": "GB/s",
                           "cores": 1, "seconds_per_step": round(dt_one / reps_one, 4),
                           "repeats": reps_one},
            "sample": f"the whole step ({B} sequences, all heads) of the same workload, NumPy "
                      f"float64: {cores} worker processes with one sequence per task and one "
                      f"BLAS thread each, repeated {reps_all} times; and on one thread, "
                      f"repeated {reps_one} times"}


def copy_mode(args, torch, debug, dev) -> int:
    """Plain device copy of --bytes, --steps times: a kernel of known traffic (reads --bytes,
    writes --bytes) for scaling the hardware byte counters."""
    src = torch.ones(args.bytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        debug.copy(dst, src)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(args.steps):
        debug.copy(dst, src)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / args.steps
    print(json.dumps({"mode": "copy", "bytes": args.bytes, "steps": args.steps,
                      "us_per_copy": round(ms * 1e3, 2),
                      "GBps_read_plus_write": round(2 * args.bytes / (ms / 1e3) / 1e9, 1)}),
          flush=True)
    return 0


def latency_mode(args, torch, pa, dev) -> int:
    """Small-batch latency rows (not the headline): the tiny workload and the two context shapes
    (32 q / 4 KV heads, D 128, bs 16, B1 L2048 and B4 L4096), each schedule run three ways:
    the eager binding (checks + launches per call), a prepared plan, and a HIP graph replaying
    the plan's launches.  With --kv fp8_e4m3 or --q-len > 1 only plans exist (the eager
    columns are null), and several query tokens run on the balanced schedule only.  Prints one
    JSON line with a row per (shape, schedule)."""
    import numpy as np

    from workloads import FP8_SCALES, make_config, make_workload

    fp8 = args.kv != "bf16"
    Q = args.q_len
    shapes = [("tiny B2 L{37,100} 4q/2kv", make_config(1, kv_format=args.kv, q_len=Q))]
    for B, L in ((1, 2048), (4, 4096)):
        shapes.append((f"context B{B} L{L} 32q/4kv D128 bs16",
                       make_workload(name="context", seq_lens=[L] * B, num_q_heads=32,
                                     num_kv_heads=4, head_dim=128, block_size=16,
                                     seed=[11, B, L], kv_format=args.kv,
                                     kv_scales=FP8_SCALES if fp8 else (1.0, 1.0), q_len=Q)))
    K = args.steps
    rows = []
    for label, wl in shapes:
        def up(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        q, k, v, bt, L = up(wl.q), up(wl.k_cache), up(wl.v_cache), up(wl.block_table), \
            up(wl.seq_lens)
        B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
        maxL = int(wl.seq_lens.max())
        out = torch.empty(wl.q.shape, dtype=torch.float32, device=dev)
        lse = torch.empty(wl.q.shape[:-1], dtype=torch.float32, device=dev)
        scheds = ("balanced",) if Q > 1 else ("unsplit", "partitioned", "fused", "balanced")
        for sched in scheds:
            P = 256 if sched in ("partitioned", "fused") else 0
            plan = pa.Plan(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, D, wl.block_size,
                           schedule=sched, partition_size=P, max_seq_len=maxL,
                           kv_dtype=args.kv, q_len=Q)
            ws = plan.workspace(dev)
            if ws is not None:
                ws.zero_()
            pmax = pa.num_partitions(maxL, P) if P else 0
            if P:
                part = torch.empty((B, Hq, pmax, D), dtype=torch.float32, device=dev)
                plse = torch.empty((B, Hq, pmax), dtype=torch.float32, device=dev)
            bws = torch.zeros(pa.balanced_workspace_size(
                pa.make_shape(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride), D)
                if sched == "balanced" else 1, dtype=torch.uint8, device=dev)

            def eager():
                if sched == "unsplit":
                    pa.decode(q, k, v, bt, L, float(wl.scale), out=out, lse=lse)
                elif sched in ("partitioned", "fused"):   # eager: decode + reduce
                    pa.decode(q, k, v, bt, L, float(wl.scale), partition_size=P,
                              max_partitions=pmax, out=part, lse=plse)
                    pa.reduce(part, plse, L, partition_size=P, out=out, lse=lse)
                else:
                    pa.decode_balanced(q, k, v, bt, L, float(wl.scale), out=out, lse=lse,
                                       workspace=bws)

            def planned():
                plan.run(q, k, v, bt, L, float(wl.scale), out=out, lse=lse, workspace=ws,
                         k_scale=wl.k_scale, v_scale=wl.v_scale)

            res = {"shape": label, "schedule": sched, "variant": plan.name, "kv_dtype": args.kv,
                   "q_len": Q}
            ways = (("plan", planned),) if (fp8 or Q > 1) else (("eager", eager), ("plan", planned))
            for name, fn in ways:
                for _ in range(10):
                    fn()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(K):
                    fn()
                t1 = time.perf_counter()
                torch.cuda.synchronize()
                t2 = time.perf_counter()
                res[f"{name}_host_us_per_call"] = round((t1 - t0) / K * 1e6, 2)
                res[f"{name}_us_per_step"] = round((t2 - t0) / K * 1e6, 2)
            # a graph of 20 consecutive steps, replayed
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                planned()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(20):
                    planned()
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, K // 20)
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            res["graph_us_per_step"] = round((time.perf_counter() - t0) / (reps * 20) * 1e6, 2)
            res["kv_bytes_per_step"] = wl.kv_bytes()
            rows.append(res)
            print(f"[latency] {res}", file=sys.stderr, flush=True)
    print(json.dumps({"mode": "latency", "steps": K, "rows": rows}), flush=True)
    return 0


class Device:
    """The GPU side of the bench: torch for memory and streams, the library for every kernel."""

    def __init__(self):
        import numpy as np
        import torch

        import paged_kv_attention_attn_amd as pa
        from paged_kv_attention_attn_amd import debug

        assert torch.cuda.is_available(), "bench.py needs a GPU"
        self.np, self.torch, self.pa, self.debug = np, torch, pa, debug
        self.dev = torch.device("cuda:0")
        self.props = torch.cuda.get_device_properties(0)
        print(f"[bench] device {self.props.name} {self.props.gcnArchName} "
              f"CUs={self.props.multi_processor_count}", file=sys.stderr, flush=True)

    def up(self, a):
        np = self.np
        a = np.ascontiguousarray(a)
        return self.torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(self.dev)


def _graph_step(torch, plan, stream, copies, steps, q, ks, vs, bt, L, wl, out, lse, sinks, ws):
    """Seconds per step of the plan's steps replayed from one HIP graph holding a step on every
    pool copy."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        plan.run(q, ks[0], vs[0], bt, L, float(wl.scale), out=out, lse=lse, sinks=sinks,
                 workspace=ws, k_scale=wl.k_scale, v_scale=wl.v_scale, stream=stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            for i in range(copies):
                plan.run(q, ks[i], vs[i], bt, L, float(wl.scale), out=out, lse=lse, sinks=sinks,
                         workspace=ws, k_scale=wl.k_scale, v_scale=wl.v_scale, stream=side)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_step = (time.perf_counter() - t0) / (reps * copies)
    del graph
    return graph_step


def measure(dv: Device, wl, *, schedule: str, partition: int, steps: int, warmup: int,
            workers: int = 0, copies=None, graph: bool = True, p_terms: int = 2) -> dict:
    """One workload on one schedule through a prepared plan (one library call per step: decode
    plus its merge).  Returns the wall time per step over ``steps`` back-to-back runs, the same
    steps replayed from a HIP graph, and the decode kernel's own duration from HIP events that
    the library records on the launch stream around it (a separate pass of the same steps)."""
    torch, pa = dv.torch, dv.pa
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    maxL = int(wl.seq_lens.max())
    pool_bytes = 2 * wl.k_cache.nbytes
    copies = copies or max(2, min(8, math.ceil(1.5 * 2 ** 30 / pool_bytes) + 1))
    q, bt, L = dv.up(wl.q), dv.up(wl.block_table), dv.up(wl.seq_lens)
    sinks = None if wl.sinks is None else dv.up(wl.sinks)
    k0, v0 = dv.up(wl.k_cache), dv.up(wl.v_cache)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    out = torch.empty(wl.q.shape, dtype=torch.float32, device=dv.dev)     # [B]([Q])[Hq][D]
    lse = torch.empty(wl.q.shape[:-1], dtype=torch.float32, device=dv.dev)
    stream = torch.cuda.current_stream(dv.dev)
    plan = pa.Plan(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, D, wl.block_size,
                   window=wl.window, schedule=schedule, partition_size=partition,
                   max_seq_len=maxL, num_workers=workers, kv_dtype=wl.kv_format, q_len=wl.q_len,
                   p_terms=p_terms)
    ws = plan.workspace(dv.dev)
    mw = re.search(r"_workers(\d+)", plan.name)
    nworkers = int(mw.group(1)) if mw else None

    def run(i):
        c = i % copies
        plan.run(q, ks[c], vs[c], bt, L, float(wl.scale), out=out, lse=lse, sinks=sinks,
                 workspace=ws, k_scale=wl.k_scale, v_scale=wl.v_scale, stream=stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps

    # the same steps from a graph: one graph holds a step on every pool copy
    graph_step = None
    if graph:
        graph_step = _graph_step(torch, plan, stream, copies, steps, q, ks, vs, bt, L, wl, out,
                                 lse, sinks, ws)

    # kernel pass: the same plan steps, with HIP events recorded on the launch stream by the
    # library right before and right after the decode kernel (its merge launch follows)
    from paged_kv_attention_attn_amd import debug

    def timed(i, ev):
        c = i % copies
        debug.plan_run_timed(plan, q, ks[c], vs[c], bt, L, float(wl.scale), out=out, lse=lse,
                             sinks=sinks, workspace=ws, k_scale=wl.k_scale, v_scale=wl.v_scale,
                             stream=stream, ev_before=ev[0], ev_after=ev[1])

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:   # creates the events
        a.record(stream)
        b.record(stream)
    for i in range(warmup):
        timed(i, evs[0])
    torch.cuda.synchronize()
    for i in range(steps):
        timed(i, evs[i])
    torch.cuda.synchronize()
    dec = sum(a.elapsed_time(b) for a, b in evs) / steps / 1e3
    res = {"schedule": schedule, "variant": plan.name, "workers": nworkers,
           "partition_size": partition or None, "kv_pool_copies": copies,
           "us_per_step": round(wall * 1e6, 2),
           "graph_us_per_step": None if graph_step is None else round(graph_step * 1e6, 2),
           "decode_us_avg": round(dec * 1e6, 3),
           "interval": "decode launch"}
    del ks, vs, k0, v0, ws, plan
    torch.cuda.empty_cache()
    return res


def gather_probe(dv: Device, chunk_bytes: int) -> dict:
    """The attainable rate of the decode kernels' access pattern: every chunk of a 2 GiB buffer
    (chunks of one 16-token tile of one KV head) read once in a random order, the best of three
    grid sizes."""
    torch = dv.torch
    buf = torch.empty(2 ** 31, dtype=torch.uint8, device=dv.dev)
    n = buf.numel() // chunk_bytes
    gen = torch.Generator(device=dv.dev).manual_seed(7)
    ids = torch.randperm(n, device=dv.dev, generator=gen).to(torch.int32)
    best = (0.0, 0)
    for wg in (512, 1024, 2048):
        sink = torch.empty(wg, dtype=torch.int32, device=dv.dev)
        for _ in range(3):
            dv.debug.gather_read(buf, chunk_bytes, ids, wg, sink)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(10):
            dv.debug.gather_read(buf, chunk_bytes, ids, wg, sink)
        s1.record()
        torch.cuda.synchronize()
        rate = buf.numel() * 10 / (s0.elapsed_time(s1) / 1e3) / 1e9
        best = max(best, (rate, wg))
    del buf, ids
    torch.cuda.empty_cache()
    return {"GBps": round(best[0], 1), "chunk_bytes": chunk_bytes, "workgroups": best[1]}


def workload_label(config: int, D: int, Hq: int, kv: str, q_len: int, seq_lens=None) -> str:
    return f"config{config}" + (f"_d{D}_hq{Hq}" if config == 3 else "") + \
        ("_fp8" if kv != "bf16" else "") + (f"_q{q_len}" if q_len > 1 else "") + \
        (f"_lens{seq_lens}" if seq_lens else "")


def row_of(wl, label: str, m: dict, roof_flops: bool = False) -> dict:
    """One workload's figures for the JSON line: µs and KV GB/s per step, fraction of the HBM
    peak, the decode kernel's µs and rate (the matrix-core rate for the query-block schedule),
    and the decode kernel's measured HBM bytes per launch where the committed counter runs hold
    them for the current kernel sources (else None)."""
    kv = wl.kv_bytes()
    r = {"workload": f"{label}: {wl.name}", **m, "kv_bytes_per_step": kv,
         "GBps": round(kv / m["us_per_step"] / 1e3, 2),
         "hbm_peak_frac": round(kv / m["us_per_step"] / 1e3 / HBM_PEAK_GBPS, 4),
         "decode_GBps": round(kv / m["decode_us_avg"] / 1e3, 2),
         "decode_hbm_peak_frac": round(kv / m["decode_us_avg"] / 1e3 / HBM_PEAK_GBPS, 4),
         "traffic": measured_traffic(label, m["schedule"])}
    if roof_flops:
        flops = attended_pairs(wl) * wl.num_q_heads * 4 * wl.head_dim
        r["decode_TFLOPs"] = round(flops / m["decode_us_avg"] / 1e6, 2)
        r["decode_mfma_peak_frac"] = round(flops / m["decode_us_avg"] / 1e6 /
                                           MFMA_BF16_PEAK_TFLOPS, 4)
    return r


# Further workloads the default run reports next to the headline: the mixed batch (window and
# sinks), the long-context step on its stated 512-token partitions and on the balanced
# schedule, the head-size sweep at group 4, the Llama-8B step with an FP8 cache, and the same
# step with 512 new tokens per sequence on the query-block schedule, with P as two bf16 terms
# (the default) and as one (the plan option PA_PLAN_P_ONE_BF16).
EXTRA_ROWS = [
    dict(config=5), dict(config=4, schedule="partitioned"), dict(config=4),
    dict(config=3, head_dim=64, q_heads=32), dict(config=3, head_dim=128, q_heads=32),
    dict(config=3, head_dim=256, q_heads=32), dict(config=2, kv="fp8_e4m3"),
    dict(config=2, q_len=512, schedule="query_blocks"),
    dict(config=2, q_len=512, schedule="query_blocks", p_terms=1),
]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--q-heads", type=int, default=None)
    ap.add_argument("--schedule", choices=["balanced", "partitioned", "unsplit",
                                           "query_blocks"],
                    default="balanced",
                    help="balanced: persistent workers + fix-up (default); partitioned: fixed "
                         "partitions + reduce; unsplit: one workgroup per (sequence, KV head); "
                         "query_blocks: one wave per (sequence, KV head, block of query "
                         "tokens) (several query tokens)")
    ap.add_argument("--partition", type=int, default=None,
                    help="partitioned schedule: partition size (default: the workload's, else "
                         "the library suggestion)")
    ap.add_argument("--workers", type=int, default=0,
                    help="balanced schedule: persistent workers (0 = device default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-rows", action="store_true",
                    help="report the headline workload only")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing (profiler runs)")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--mode", choices=["decode", "copy", "latency"], default="decode",
                    help="copy: run only the plain copy kernel on --bytes (counter calibration); "
                         "latency: small-batch rows, eager vs prepared plan vs graph replay")
    ap.add_argument("--bytes", type=int, default=1 << 30)
    ap.add_argument("--kv", choices=["bf16", "fp8_e4m3"], default="bf16",
                    help="KV cache format")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (> 1: causal; balanced or query_blocks)")
    ap.add_argument("--p-terms", type=int, choices=[1, 2], default=2,
                    help="query-block schedule: P as two bf16 terms (default) or one "
                         "(PA_PLAN_P_ONE_BF16)")
    ap.add_argument("--seq-lens", default=None,
                    help="replace the workload's lengths (its head geometry kept): 'BxL' for B "
                         "sequences of L tokens, or a comma-separated list")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this "
              "single-GPU decode kernel build", file=sys.stderr)
        return 2

    from workloads import make_config

    def workload(config, head_dim=128, q_heads=None, kv="bf16", q_len=1, seq_lens=None):
        kw = {}
        if config == 3:
            kw = dict(head_dim=head_dim, num_q_heads=q_heads or 32)
        if seq_lens:
            if "x" in seq_lens:
                nb, ln = (int(x) for x in seq_lens.split("x"))
                kw["seq_lens"] = [ln] * nb
            else:
                kw["seq_lens"] = [int(x) for x in seq_lens.split(",")]
        return make_config(config, kv_format=kv, q_len=q_len, **kw)

    # the headline workload, and the oracle baseline before anything touches the GPU
    wl = None
    if args.mode == "decode":
        wl = workload(args.config, args.head_dim, args.q_heads, args.kv, args.q_len,
                      args.seq_lens)
    cpu = None
    if wl is not None and not args.no_cpu_baseline:
        print("[bench] oracle baseline on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    dv = Device()
    if args.mode == "copy":
        return copy_mode(args, dv.torch, dv.debug, dv.dev)
    if args.mode == "latency":
        return latency_mode(args, dv.torch, dv.pa, dv.dev)

    def partition_of(w, schedule):
        if schedule != "partitioned":
            return 0
        if args.partition is not None:
            return args.partition
        return w.partition_size or dv.pa.suggest_partition_size(
            w.num_seqs, w.num_kv_heads, int(w.seq_lens.max()), w.block_size,
            dv.props.multi_processor_count)

    D, Hq = wl.head_dim, wl.num_q_heads
    P = partition_of(wl, args.schedule)
    kv_bytes = wl.kv_bytes()
    print(f"[bench] {wl.name}: kv_bytes/step={kv_bytes / 1e6:.1f} MB, schedule={args.schedule}, "
          f"P={P}", file=sys.stderr, flush=True)
    m = measure(dv, wl, schedule=args.schedule, partition=P, steps=args.steps,
                warmup=args.warmup, workers=args.workers, copies=args.copies,
                graph=not args.no_graph, p_terms=args.p_terms)
    print(f"[bench] headline {m}", file=sys.stderr, flush=True)
    label = workload_label(args.config, D, Hq, args.kv, args.q_len, args.seq_lens) + \
        ("_p1" if args.p_terms == 1 else "")
    qblocks = args.schedule == "query_blocks"
    # chunks of one 16-token tile of one KV head (the probe takes 2 to 8 KiB; an FP8 tile at
    # head_dim 64 is 1 KiB and is compared with 2 KiB chunks)
    probe = gather_probe(dv, min(max(16 * D * (1 if args.kv != "bf16" else 2), 2048), 8192))
    print(f"[bench] gather probe {probe}", file=sys.stderr, flush=True)

    us = m["us_per_step"]
    dec_s = m["decode_us_avg"] / 1e6
    achieved = kv_bytes / dec_s / 1e9
    value = kv_bytes / (us / 1e6) / 1e9
    res = {
        "metric": METRIC if args.kv == "bf16" else METRIC.replace("bf16 d=128",
                                                                  "FP8 E4M3 KV d=128"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "us_per_step": us,
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "graph_us_per_step": m["graph_us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{label}: {wl.name}" +
                        (f" (lengths replaced: {args.seq_lens})" if args.seq_lens else ""),
            "batch": wl.num_seqs, "q_heads": Hq, "kv_heads": wl.num_kv_heads, "head_dim": D,
            "block_size": wl.block_size, "window": wl.window,
            "sinks": wl.sinks is not None, "seq_len_sum": int(wl.seq_lens.sum()),
            "max_seq_len": int(wl.seq_lens.max()), "schedule": args.schedule,
            "kv_dtype": args.kv, "q_len": args.q_len, "partition_size": P or None,
            "workers": m["workers"], "kv_bytes_per_step": kv_bytes, "variant": m["variant"],
            "kv_pool_copies": m["kv_pool_copies"], "parallelism": "none (1 GPU)",
            "timing": "value and us_per_step: wall clock over back-to-back prepared-plan runs "
                      "(one library call per step: decode + merge); graph_us_per_step: the same "
                      "steps replayed from a HIP graph; roofline: HIP events the library records "
                      "on the launch stream right before and after the decode kernel, in a "
                      "second pass of the same plan steps",
            "device": {"name": dv.props.name, "arch": dv.props.gcnArchName,
                       "hip": str(dv.torch.version.hip), "torch": dv.torch.__version__},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": m["variant"],
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(label, args.schedule),
            "decode_us_avg": m["decode_us_avg"],
            "interval": m["interval"],
            "algorithmic_bytes_per_launch": kv_bytes,
            "attainable_gather_read_GBps": probe["GBps"],
            "attainable_probe": probe,
            "frac_of_attainable": round(achieved / probe["GBps"], 4),
        },
    }
    if qblocks:
        # query blocks with many tokens per sequence are a dense contraction: 4 D flops per
        # attended (query token, key) pair and query head (q.k and P.V, 2 D each)
        flops = attended_pairs(wl) * Hq * 4 * D
        res["roofline"].update({
            "bound": "mfma", "achieved": round(flops / dec_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / dec_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": flops, "kv_read_GBps": round(achieved, 2)})
        for key in ("attainable_gather_read_GBps", "attainable_probe", "frac_of_attainable"):
            res["roofline"].pop(key)
    del wl

    default_run = (args.config == 2 and args.schedule == "balanced" and args.kv == "bf16" and
                   args.q_len == 1 and not args.seq_lens and not args.workers)
    if default_run and not args.no_extra_rows:
        rows = []
        for spec in EXTRA_ROWS:
            sched = spec.get("schedule", "balanced")
            w = workload(spec["config"], spec.get("head_dim", 128), spec.get("q_heads"),
                         spec.get("kv", "bf16"), spec.get("q_len", 1))
            lab = workload_label(spec["config"], w.head_dim, w.num_q_heads, w.kv_format,
                                 w.q_len) + ("_p1" if spec.get("p_terms", 2) == 1 else "")
            mm = measure(dv, w, schedule=sched, partition=partition_of(w, sched),
                         steps=args.steps, warmup=args.warmup, graph=not args.no_graph,
                         p_terms=spec.get("p_terms", 2))
            r = row_of(w, lab, mm, roof_flops=sched == "query_blocks")
            print(f"[bench] row {r}", file=sys.stderr, flush=True)
            rows.append(r)
            del w
        res["workloads"] = rows
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Decode-step benchmark: one paged-attention decode step (decode + split-KV reduce) over a
synthetic Llama-8B-shaped batch, on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--partition P]

Prints ONE JSON line.  value = algorithmic KV bytes per step / wall time per step (GB/s), with
inputs resident in HBM; the timed region is K back-to-back steps bracketed by synchronisation.
Several identical copies of the KV pools are rotated across steps so that no step finds its KV
in the 256 MB last-level (MALL) cache.  roofline.achieved divides the same KV bytes by the
decode kernel's own average duration (HIP events recorded on the launch stream around every
decode launch of the timed region).  cpu_baseline times the fp64 oracle on the host.
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


def cpu_baseline(wl, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle on this host, one thread, over the whole step's batch, repeated until at
    least ``min_seconds`` have passed; the value is the mean rate."""
    from threadpoolctl import threadpool_limits

    from oracle import ref

    reps, dt = 0, 0.0
    with threadpool_limits(1):
        while dt < min_seconds:
            t0 = time.perf_counter()
            fn = ref.decode_multi if wl.q_len > 1 else ref.decode
            fn(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
               wl.block_size, window=wl.window, sinks=wl.sinks, kv_format=wl.kv_format,
               k_scale=wl.k_scale, v_scale=wl.v_scale)
            dt += time.perf_counter() - t0
            reps += 1
    return {"value": round(wl.kv_bytes() * reps / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds_per_step": round(dt / reps, 3), "repeats": reps,
            "cpu_model": _cpu_model(),
            "sample": f"the whole step ({wl.num_seqs} sequences, all heads) of the same "
                      f"workload, NumPy float64, 1 BLAS thread, repeated {reps} times"}


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
                         "tokens), through a prepared plan (several query tokens)")
    ap.add_argument("--partition", type=int, default=None,
                    help="partitioned schedule: partition size (default: library suggestion)")
    ap.add_argument("--workers", type=int, default=0,
                    help="balanced schedule: persistent workers (0 = device default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=None)
    ap.add_argument("--mode", choices=["decode", "copy", "latency"], default="decode",
                    help="copy: run only the plain copy kernel on --bytes (counter calibration); "
                         "latency: small-batch rows, eager vs prepared plan vs graph replay")
    ap.add_argument("--bytes", type=int, default=1 << 30)
    ap.add_argument("--kv", choices=["bf16", "fp8_e4m3"], default="bf16",
                    help="KV cache format; fp8_e4m3 runs through a prepared plan (the timed "
                         "kernel interval then spans the decode and merge launches)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (> 1: causal, balanced schedule, through a "
                         "prepared plan like --kv fp8_e4m3)")
    ap.add_argument("--seq-lens", default=None,
                    help="replace the workload's lengths (its head geometry kept): 'BxL' for B "
                         "sequences of L tokens, or a comma-separated list")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this "
              "single-GPU decode kernel build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_attention_attn_amd as pa
    from paged_kv_attention_attn_amd import debug
    from workloads import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    print(f"[bench] device {props.name} {props.gcnArchName} CUs={props.multi_processor_count}",
          file=sys.stderr, flush=True)

    if args.mode == "copy":
        return copy_mode(args, torch, debug, dev)
    if args.mode == "latency":
        return latency_mode(args, torch, pa, dev)

    kw = {}
    if args.config == 3:
        kw = dict(head_dim=args.head_dim, num_q_heads=args.q_heads or 32)
    if args.seq_lens:
        if "x" in args.seq_lens:
            nb, ln = (int(x) for x in args.seq_lens.split("x"))
            kw["seq_lens"] = [ln] * nb
        else:
            kw["seq_lens"] = [int(x) for x in args.seq_lens.split(",")]
    wl = make_config(args.config, kv_format=args.kv, q_len=args.q_len, **kw)
    fp8 = args.kv != "bf16"
    qblocks = args.schedule == "query_blocks"
    planned = fp8 or args.q_len > 1 or qblocks
    B, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    maxL = int(wl.seq_lens.max())
    if args.schedule == "unsplit" or qblocks:
        P = 0
    elif args.schedule == "partitioned":
        P = args.partition
        if P is None:
            P = wl.partition_size or pa.suggest_partition_size(B, wl.num_kv_heads, maxL,
                                                               wl.block_size,
                                                               props.multi_processor_count)
    else:
        P = -1
    pmax = pa.num_partitions(maxL, P) if P > 0 else 0
    kv_bytes = wl.kv_bytes()
    pool_bytes = 2 * wl.k_cache.nbytes
    copies = args.copies or max(2, min(8, math.ceil(1.5 * 2 ** 30 / pool_bytes) + 1))
    print(f"[bench] {wl.name}: kv_bytes/step={kv_bytes / 1e6:.1f} MB, P={P}, pmax={pmax}, "
          f"pool={pool_bytes / 1e6:.0f} MB x {copies} copies", file=sys.stderr, flush=True)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    q, bt, L = up(wl.q), up(wl.block_table), up(wl.seq_lens)
    sinks = None if wl.sinks is None else up(wl.sinks)
    k0, v0 = up(wl.k_cache), up(wl.v_cache)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    out = torch.empty(wl.q.shape, dtype=torch.float32, device=dev)      # [B]([Q])[Hq][D]
    lse = torch.empty(wl.q.shape[:-1], dtype=torch.float32, device=dev)
    if P > 0:
        part = torch.empty((B, Hq, pmax, D), dtype=torch.float32, device=dev)
        plse = torch.empty((B, Hq, pmax), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    shape = pa.make_shape(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, max(P, 0), pmax)
    workers = args.workers
    plan = None
    if planned:
        plan = pa.Plan(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, D, wl.block_size,
                       window=wl.window, schedule=args.schedule, partition_size=max(P, 0),
                       max_seq_len=maxL, num_workers=workers, kv_dtype=args.kv,
                       q_len=args.q_len)
        plan_ws = plan.workspace(dev)
        variant = plan.name
        if P < 0:
            workers = int(variant.split("workers")[1].split()[0])
        if qblocks:
            workers = None
    elif P < 0:
        workers = workers or pa.balanced_default_workers(D, Hq // wl.num_kv_heads)
        ws = torch.empty(pa.balanced_workspace_size(shape, D, workers), dtype=torch.uint8,
                         device=dev)
        path = (pa.variant_name(shape, D, wl.block_size) or "pa_decode_?").split("_")[2]
        variant = f"pa_balanced_{path}" \
                  f"_d{D}_g{Hq // wl.num_kv_heads}_workers{workers}"
    else:
        variant = pa.variant_name(shape, D, wl.block_size)

    # one decode step = the decode kernel launch, then its merge launch (if any); events mark the
    # end of the decode launch so its own duration can be read
    def step(i, ev=None):
        c = i % copies
        if ev is not None:
            ev[0].record(stream)
        if plan is not None:
            plan.run(q, ks[c], vs[c], bt, L, float(wl.scale), out=out, lse=lse, sinks=sinks,
                     workspace=plan_ws, k_scale=wl.k_scale, v_scale=wl.v_scale, stream=stream)
        elif P > 0:
            pa.decode(q, ks[c], vs[c], bt, L, float(wl.scale), window=wl.window, sinks=sinks,
                      partition_size=P, max_partitions=pmax, out=part, lse=plse, stream=stream)
        elif P == 0:
            pa.decode(q, ks[c], vs[c], bt, L, float(wl.scale), window=wl.window, sinks=sinks,
                      out=out, lse=lse, stream=stream)
        else:
            pa.decode_balanced(q, ks[c], vs[c], bt, L, float(wl.scale), window=wl.window,
                               sinks=sinks, out=out, lse=lse, workspace=ws, num_workers=workers,
                               merge=False, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if plan is not None:
            pass
        elif P > 0:
            pa.reduce(part, plse, L, partition_size=P, out=out, lse=lse, stream=stream)
        elif P < 0:
            pa.reduce_balanced(L, out, lse, shape=shape, head_dim=D, block_size=wl.block_size,
                               window=wl.window, sinks=sinks, workspace=ws,
                               num_workers=workers, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, HIP events on the launch stream around each decode launch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    dec_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3
    value = kv_bytes / (wall / args.steps) / 1e9
    achieved = kv_bytes / dec_avg_s / 1e9

    # attainable streaming read on this device (context for the roofline fraction)
    probe = torch.empty(2 ** 31, dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    for _ in range(3):
        debug.stream_read(probe, 4096, sink)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(10):
        debug.stream_read(probe, 4096, sink)
    s1.record(stream)
    torch.cuda.synchronize()
    attainable = probe.numel() * 10 / (s0.elapsed_time(s1) / 1e3) / 1e9
    del probe

    workload = f"config{args.config}" + (f"_d{D}_hq{Hq}" if args.config == 3 else "") + \
        ("_fp8" if fp8 else "") + (f"_q{args.q_len}" if args.q_len > 1 else "") + \
        (f"_lens{args.seq_lens}" if args.seq_lens else "")
    traffic = measured_traffic(workload, args.schedule)
    res = {
        "metric": METRIC if not fp8 else METRIC.replace("bf16 d=128", "FP8 E4M3 KV d=128"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{workload}: {wl.name}" +
                        (f" (lengths replaced: {args.seq_lens})" if args.seq_lens else ""),
            "batch": B, "q_heads": Hq, "kv_heads": wl.num_kv_heads, "head_dim": D,
            "block_size": wl.block_size, "window": wl.window,
            "sinks": wl.sinks is not None, "seq_len_sum": int(wl.seq_lens.sum()),
            "max_seq_len": maxL, "schedule": args.schedule, "kv_dtype": args.kv,
            "q_len": args.q_len,
            "partition_size": P if P > 0 else None,
            "workers": workers if P < 0 else None, "kv_bytes_per_step": kv_bytes,
            "variant": variant, "kv_pool_copies": copies, "parallelism": "none (1 GPU)",
            "device": {"name": props.name, "arch": props.gcnArchName,
                       "hip": str(torch.version.hip), "torch": torch.__version__},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": variant,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "decode_us_avg": round(dec_avg_s * 1e6, 3),
            "interval": "decode and merge launches" if planned else "decode launch",
            "algorithmic_bytes_per_launch": kv_bytes,
            "attainable_stream_read_GBps": round(attainable, 1),
            "frac_of_attainable": round(achieved / attainable, 4),
        },
    }
    if qblocks:
        # query blocks with many tokens per sequence are a dense contraction: 4 D flops per
        # attended (query token, key) pair and query head (q.k and P.V, 2 D each)
        flops = attended_pairs(wl) * Hq * 4 * D
        res["roofline"].update({
            "bound": "mfma", "achieved": round(flops / dec_avg_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / dec_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": flops,
            "kv_read_GBps": round(achieved, 2)})
        for key in ("attainable_stream_read_GBps", "frac_of_attainable"):
            res["roofline"].pop(key)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

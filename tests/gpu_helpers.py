"""Shared helpers for the GPU parity tests: move a seeded workload to the device, run the HIP
path through the C ABI (via the thin binding), and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_attention_attn_amd as pa
from oracle import ref
from tests.oracle_rows import oracle_multi_triples  # noqa: F401 (re-exported)

# Contract: max abs error <= 3e-2 against the fp64 oracle (bf16 inputs, fp32 accumulation).
TOL = 3e-2
# Regression gates, far tighter than the contract: fp32 accumulation lands ~1e-6 from fp64.
REG_ABS = 1e-3
REG_NMSE = 5e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(wl):
    d = torch.device("cuda")
    kv = np.uint8 if wl.kv_format == "fp8_e4m3" else np.int16   # raw codes / bf16 bits
    t = dict(
        q=torch.from_numpy(np.ascontiguousarray(wl.q).view(np.int16)).to(d),
        k=torch.from_numpy(np.ascontiguousarray(wl.k_cache).view(kv)).to(d),
        v=torch.from_numpy(np.ascontiguousarray(wl.v_cache).view(kv)).to(d),
        bt=torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(d),
        L=torch.from_numpy(np.ascontiguousarray(wl.seq_lens)).to(d),
        sinks=None if wl.sinks is None else torch.from_numpy(wl.sinks).to(d),
    )
    torch.cuda.synchronize()
    return t


def max_len(wl) -> int:
    return int(wl.seq_lens.max()) if wl.num_seqs else 0


BALANCED = -1   # partition_size value that selects the balanced schedule in run_gpu


def run_gpu(wl, t, partition_size: int = 0, max_partitions=None, num_workers: int = 0):
    """One decode step through the ABI; returns (out, lse) as NumPy float64.  Output buffers (and
    the balanced workspace) are NaN-poisoned first so an unwritten element cannot pass.
    partition_size: 0 unsplit, > 0 fixed partitions + reduce, BALANCED the balanced schedule."""
    B, Hq, D = wl.q.shape
    dev = t["q"].device
    if partition_size == BALANCED:
        out = torch.full((B, Hq, D), float("nan"), device=dev)
        lse = torch.full((B, Hq), float("nan"), device=dev)
        shape = pa.make_shape(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride)
        nbytes = pa.balanced_workspace_size(shape, D, num_workers)
        ws = torch.full((nbytes // 4 + 1,), float("nan"), device=dev)
        pa.decode_balanced(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                           window=wl.window, sinks=t["sinks"], out=out, lse=lse, workspace=ws,
                           num_workers=num_workers)
    elif partition_size == 0:
        out = torch.full((B, Hq, D), float("nan"), device=dev)
        lse = torch.full((B, Hq), float("nan"), device=dev)
        pa.decode(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale), window=wl.window,
                  sinks=t["sinks"], out=out, lse=lse)
    else:
        pmax = max_partitions or pa.num_partitions(max_len(wl), partition_size)
        part = torch.full((B, Hq, pmax, D), float("nan"), device=dev)
        plse = torch.full((B, Hq, pmax), float("nan"), device=dev)
        pa.decode(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale), window=wl.window,
                  sinks=t["sinks"], partition_size=partition_size, max_partitions=pmax,
                  out=part, lse=plse)
        out = torch.full((B, Hq, D), float("nan"), device=dev)
        lse = torch.full((B, Hq), float("nan"), device=dev)
        pa.reduce(part, plse, t["L"], partition_size=partition_size, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_full(wl):
    if wl.q_len > 1:
        return ref.decode_multi(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                wl.scale, wl.block_size, window=wl.window, sinks=wl.sinks,
                                kv_format=wl.kv_format, k_scale=wl.k_scale, v_scale=wl.v_scale)
    return ref.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                      wl.block_size, window=wl.window, sinks=wl.sinks, kv_format=wl.kv_format,
                      k_scale=wl.k_scale, v_scale=wl.v_scale)


def compare(got_out, got_lse, exp_out, exp_lse, tag: str, strict: bool = True) -> dict:
    """Element-wise comparison; asserts the contract (and the regression gates when strict)."""
    assert got_out.shape == exp_out.shape, (tag, got_out.shape, exp_out.shape)
    assert np.isfinite(got_out).all(), f"{tag}: non-finite output at " \
        f"{np.argwhere(~np.isfinite(got_out))[:4].tolist()}"
    err = np.abs(got_out - exp_out)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    emax = float(err[i])
    denom = float(np.sum(exp_out ** 2))
    nmse = float(np.sum((got_out - exp_out) ** 2) / denom) if denom > 0 else 0.0
    # lse: -inf where the oracle says so, else within tolerance
    ninf = np.isneginf(exp_lse)
    assert np.array_equal(np.isneginf(got_lse), ninf), f"{tag}: -inf lse pattern differs"
    fin = ~ninf
    assert np.isfinite(got_lse[fin]).all(), f"{tag}: non-finite lse"
    lerr = float(np.abs(got_lse[fin] - exp_lse[fin]).max()) if fin.any() else 0.0
    log(f"[parity] {tag}: max|out err|={emax:.3e} at {tuple(int(x) for x in i)} "
        f"nmse={nmse:.3e} max|lse err|={lerr:.3e}")
    assert emax <= TOL, f"{tag}: out error {emax} > {TOL} at {i}"
    assert lerr <= TOL, f"{tag}: lse error {lerr} > {TOL}"
    if strict:
        assert emax <= REG_ABS, f"{tag}: out error {emax} above the regression gate {REG_ABS}"
        assert lerr <= REG_ABS, f"{tag}: lse error {lerr} above the regression gate {REG_ABS}"
        assert nmse <= REG_NMSE, f"{tag}: nmse {nmse}"
    return dict(max_abs=emax, nmse=nmse, lse_max_abs=lerr)


def cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def bench_partition(wl) -> int:
    """Partition size the bench uses for this workload."""
    if wl.partition_size:
        return wl.partition_size
    return pa.suggest_partition_size(wl.num_seqs, wl.num_kv_heads, max_len(wl), wl.block_size,
                                     cus())


def finite_rows(x):
    return np.isfinite(x).all(axis=-1)


# ---------------------------------------------------------------------------------------------
# prepared decode steps (plans)
# ---------------------------------------------------------------------------------------------
def make_plan(wl, schedule, partition_size=256, num_workers=0):
    return pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule=schedule,
                   partition_size=partition_size, max_seq_len=max_len(wl),
                   num_workers=num_workers, kv_dtype=wl.kv_format, q_len=wl.q_len)


def counter_bytes(wl):
    """The fused schedule's merge counters: the last 256-byte-aligned section of its workspace."""
    return (4 * wl.num_seqs * wl.num_kv_heads + 255) // 256 * 256


def run_plan(plan, wl, t, workspace=None):
    """One step through paged_attn_plan_run into NaN-filled outputs (and, unless a workspace is
    given, a workspace whose non-counter bytes are 0xFF); returns (out, lse) as float64."""
    fused = "last partition" in plan.name
    out = torch.full(wl.q.shape, float("nan"), device="cuda")      # [B]([Q])[Hq][D]
    lse = torch.full(wl.q.shape[:-1], float("nan"), device="cuda")
    ws = workspace if workspace is not None else plan.workspace("cuda")
    if ws is not None and workspace is None:
        # stale contents must not matter (except the fused counters, which start at zero)
        ws[:ws.numel() - (counter_bytes(wl) if fused else 0)].fill_(0xFF)
    plan.run(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale), out=out, lse=lse,
             sinks=t["sinks"], workspace=ws, k_scale=wl.k_scale, v_scale=wl.v_scale)
    torch.cuda.synchronize()
    if fused:
        assert int(torch.count_nonzero(ws[ws.numel() - counter_bytes(wl):])) == 0, \
            "merge counters not back at zero"
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

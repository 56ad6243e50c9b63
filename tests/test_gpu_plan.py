"""GPU tests of prepared decode steps (plans): parity with the fp64 oracle through
paged_attn_plan_run for every schedule, NaN inputs inside the attended range, and HIP-graph
capture and replay of a run."""
from __future__ import annotations

import re

import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from workloads import FP8_QNAN, make_config, make_workload

from gpu_helpers import compare, log, make_plan, oracle_full, run_plan, to_dev

pytestmark = pytest.mark.gpu

SCHEDULES = ["unsplit", "partitioned", "balanced", "fused"]


def context_workload(B, L):
    """The small-batch context shapes: 32 q / 4 KV heads, D 128, block size 16."""
    return make_workload(name=f"context B{B} L{L}", seq_lens=[L] * B, num_q_heads=32,
                         num_kv_heads=4, head_dim=128, block_size=16, seed=[11, B, L],
                         poison=True)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_plan_config1(schedule):
    wl = make_config(1, poison=True)
    plan = make_plan(wl, schedule, partition_size=32)
    log(f"[plan] {plan.name}")
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"plan cfg1 {schedule}")


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_plan_config5_window_sinks(schedule):
    wl = make_config(5, poison=True)
    plan = make_plan(wl, schedule, partition_size=1024)
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"plan cfg5 {schedule}")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("B,L", [(1, 2048), (4, 4096)])
def test_plan_context_shapes(B, L, schedule):
    wl = context_workload(B, L)
    plan = make_plan(wl, schedule, partition_size=256)
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"plan context B{B} L{L} {schedule}")


def test_plan_empty_batch_is_a_no_op():
    wl = make_config(1)
    plan = pa.Plan(0, 4, 2, wl.num_blocks, wl.stride, 128, 16, schedule="balanced")
    x = torch.zeros(1, device="cuda")
    plan.run(x, x, x, x, x, 0.1, out=x, workspace=plan.workspace("cuda"))
    torch.cuda.synchronize()
    assert float(x.item()) == 0.0


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_nan_in_attended_row(schedule, kv, which):
    """A NaN (bf16 0x7FC0, or the FP8 code 0x7F) inside the attended range of one (sequence, KV
    head): in K the oracle gives NaN outputs and LSEs for that KV head's query heads, in V NaN
    in the one output dimension it sits in; the kernels must give NaN in exactly those places
    and match everywhere else."""
    wl = make_workload(name="nan", seq_lens=[200, 90, 333], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[22], poison=True, kv_format=kv,
                       kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0))
    cache = wl.k_cache if which == "k" else wl.v_cache
    tok = 77                                     # sequence 1, KV head 1, inside its 90 tokens
    cache[wl.block_table[1, tok // 16], 1, tok % 16, 5] = \
        FP8_QNAN if kv != "bf16" else np.uint16(0x7FC0)
    exp_o, exp_l = oracle_full(wl)
    if which == "k":
        assert np.isnan(exp_o[1, 4:8]).all() and np.isnan(exp_l[1, 4:8]).all()
        assert np.isnan(exp_o).sum() == 4 * 128
    else:
        assert np.isnan(exp_o[1, 4:8, 5]).all() and np.isnan(exp_o).sum() == 4
        assert not np.isnan(exp_l).any()
    got_o, got_l = run_plan(make_plan(wl, schedule, partition_size=32), wl, to_dev(wl))
    bad_o = np.argwhere(np.isnan(got_o) != np.isnan(exp_o))
    bad_l = np.argwhere(np.isnan(got_l) != np.isnan(exp_l))
    assert bad_o.size == 0, f"NaN pattern of out differs at {bad_o[:4].tolist()} " \
        f"({len(bad_o)} places)"
    assert bad_l.size == 0, f"NaN pattern of lse differs at {bad_l[:4].tolist()}"
    ok = ~np.isnan(exp_o)
    assert np.abs(got_o[ok] - exp_o[ok]).max() <= 1e-3
    okl = ~np.isnan(exp_l)
    assert np.abs(got_l[okl] - exp_l[okl]).max() <= 1e-3


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_plan_graph_replay(schedule):
    """A run captured in a graph and replayed five times, with the inputs changed in place and
    eager runs and synchronisations between replays: every replay equals the eager run bit for
    bit, and one of them the oracle."""
    wl = context_workload(4, 4096)
    t = to_dev(wl)
    plan = make_plan(wl, schedule, partition_size=256)
    B, Hq, D = wl.q.shape
    ws = plan.workspace("cuda")
    out = torch.zeros((B, Hq, D), device="cuda")
    lse = torch.zeros((B, Hq), device="cuda")
    args = (t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(*args, out=out, lse=lse, workspace=ws)     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(*args, out=out, lse=lse, workspace=ws)
    q0 = t["q"].clone()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for r in range(5):
        # new query values (bf16 bit patterns of N(0,1) draws), written in place
        t["q"].copy_(torch.randn(q0.shape, device="cuda", generator=gen)
                     .to(torch.bfloat16).view(torch.int16))
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref_out = torch.full_like(out, float("nan"))
        ref_lse = torch.full_like(lse, float("nan"))
        ws_ref = plan.workspace("cuda")
        plan.run(*args, out=ref_out, lse=ref_lse, workspace=ws_ref)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref_out) and torch.equal(got[1], ref_lse), f"replay {r}"
        if r == 4:
            wl.q[...] = t["q"].cpu().numpy().view(np.uint16)
            compare(got[0].cpu().numpy().astype(np.float64),
                    got[1].cpu().numpy().astype(np.float64), *oracle_full(wl),
                    f"graph replay {schedule}")
    t["q"].copy_(q0)


def test_plan_length_bound_caps_workers_and_a_violated_bound_stays_correct():
    wl = make_config(1, poison=True)
    B, Hq, D = wl.q.shape
    capped = pa.Plan(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, D, wl.block_size,
                     schedule="balanced", max_seq_len=100)
    m = re.search(r"_workers(\d+)", capped.name)
    assert m and int(m.group(1)) <= 8, capped.name
    low = pa.Plan(B, Hq, wl.num_kv_heads, wl.num_blocks, wl.stride, D, wl.block_size,
                  schedule="balanced", max_seq_len=16)    # below the real lengths (37, 100)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_plan(capped, wl, t), *exp, f"plan {capped.name}")
    compare(*run_plan(low, wl, t), *exp, f"plan {low.name} (bound below the lengths)")


def auto_workload(case):
    if case == "tiny":
        return make_config(1, poison=True), "unsplit"
    if case == "context":
        return context_workload(1, 2048), "partitioned"
    if case == "llama":
        return make_config(2, poison=True), "balanced"
    if case == "mixed":
        return make_config(5, poison=True, seq_lens=[5000, 17, 9000, 4096, 1, 300, 0]), \
            "partitioned"
    Q = {"q4": 4, "q16": 16}[case]
    wl = make_workload(name=f"auto {case}", seq_lens=[3000, 17, 600, Q - 1], num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=16, seed=[12, Q],
                       with_sinks=True, poison=True, q_len=Q)
    return wl, ("balanced" if Q == 4 else "query_blocks")


@pytest.mark.parametrize("case", ["tiny", "context", "llama", "mixed", "q4", "q16"])
def test_auto_schedule(case):
    """schedule="auto" takes the library's suggestion for the sizes (on this device) and runs
    it: the expected schedule, and the oracle's results."""
    wl, expected = auto_workload(case)
    plan = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule="auto",
                   max_seq_len=int(wl.seq_lens.max()), q_len=wl.q_len)
    log(f"[auto] {case}: {plan.schedule} {plan.name}")
    assert plan.schedule == expected
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"auto {case} -> {plan.name}")


def _timed_case(case):
    if case == "qblocks_split":   # two sequences: key splits and their merge
        return make_workload(name="timed qblocks split", seq_lens=[3000, 2100], num_q_heads=8,
                             num_kv_heads=2, head_dim=128, block_size=16, seed=[5, 1],
                             poison=True, q_len=40), "query_blocks"
    if case == "qblocks":
        return make_workload(name="timed qblocks", seq_lens=[300, 17, 1000, 41] * 16,
                             num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                             seed=[5, 2], poison=True, q_len=40), "query_blocks"
    if case == "fp8":
        return make_workload(name="timed fp8", seq_lens=[700, 1, 4000, 33], num_q_heads=16,
                             num_kv_heads=4, head_dim=128, block_size=16, seed=[5, 3],
                             poison=True, kv_format="fp8_e4m3",
                             kv_scales=(0.0625, 0.05)), "balanced"
    return make_config(5, poison=True), case


@pytest.mark.parametrize("case", SCHEDULES + ["fp8", "qblocks", "qblocks_split"])
def test_plan_run_timed_matches_run(case):
    """The timed run launches what run() launches (bit-identical outputs) and its events
    bracket a kernel of positive duration that is no longer than the whole step."""
    from paged_kv_attention_attn_amd import debug
    wl, schedule = _timed_case(case)
    plan = make_plan(wl, schedule, partition_size=1024)
    log(f"[timed] {case} {plan.name}")
    t = to_dev(wl)
    ws = plan.workspace("cuda")
    want = run_plan(plan, wl, t, workspace=ws)
    out = torch.full(wl.q.shape, float("nan"), device="cuda")
    lse = torch.full(wl.q.shape[:-1], float("nan"), device="cuda")
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for x in e:
        x.record()
    e[2].record()
    debug.plan_run_timed(plan, t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                         out=out, lse=lse, sinks=t["sinks"], workspace=ws, k_scale=wl.k_scale,
                         v_scale=wl.v_scale, ev_before=e[0], ev_after=e[1])
    e[3].record()
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want[0].astype(np.float32), equal_nan=True)
    assert np.array_equal(lse.cpu().numpy(), want[1].astype(np.float32), equal_nan=True)
    kernel_ms, step_ms = e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])
    assert 0.0 < kernel_ms <= step_ms, (kernel_ms, step_ms)
    with pytest.raises(ValueError):
        debug.plan_run_timed(plan, t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                             out=out, ev_before=torch.cuda.Event(enable_timing=True),
                             ev_after=e[1], sinks=t["sinks"], workspace=ws)

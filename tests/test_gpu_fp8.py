"""GPU parity of the FP8 E4M3 KV-cache path (per-tensor K and V scales) against the fp64 oracle,
through paged_attn_plan_run, for every schedule: the workload shapes, the edge lengths, window
and sinks, NaN codes outside the attended range, negative scales and graph replay (NaN codes
inside it are covered with the bf16 ones by the plan tests).

An E4M3 value is exact in bf16, so the kernels' arithmetic is that of the bf16 path and the same
bars hold: the 3e-2 contract and the 1e-3 regression gate on the output and the LSE."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from workloads import make_config, make_workload

from gpu_helpers import bench_partition, compare, log, make_plan, oracle_full, run_plan, to_dev

pytestmark = pytest.mark.gpu

FP8 = "fp8_e4m3"
SCHEDULES = ["unsplit", "partitioned", "balanced", "fused"]


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_fp8_config1(schedule):
    wl = make_config(1, poison=True, kv_format=FP8)
    plan = make_plan(wl, schedule, partition_size=32)
    log(f"[fp8] {plan.name}")
    assert "fp8" in plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"fp8 cfg1 {schedule}")


def test_fp8_config2_bench_launch():
    """The decode-batch workload at full size, balanced with the device's default workers (the
    bench's launch), and partitioned at the bench's partition size."""
    wl = make_config(2, poison=True, kv_format=FP8)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_plan(make_plan(wl, "balanced"), wl, t), *exp, "fp8 cfg2 balanced")
    P = bench_partition(wl)
    compare(*run_plan(make_plan(wl, "partitioned", partition_size=P), wl, t), *exp,
            f"fp8 cfg2 partitioned P={P}")


@pytest.mark.parametrize("schedule", ["balanced", "partitioned", "unsplit"])
def test_fp8_config5_window_sinks(schedule):
    wl = make_config(5, poison=True, kv_format=FP8)
    plan = make_plan(wl, schedule, partition_size=bench_partition(wl))
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"fp8 cfg5 {schedule}")


def test_fp8_config4_long_context():
    wl = make_config(4, kv_format=FP8)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_plan(make_plan(wl, "partitioned", partition_size=512), wl, t), *exp,
            "fp8 cfg4 partitioned P=512")
    compare(*run_plan(make_plan(wl, "balanced"), wl, t), *exp, "fp8 cfg4 balanced")


@pytest.mark.parametrize("D,hq", [(D, hq) for D in (64, 128, 256) for hq in (8, 32, 64)])
def test_fp8_config3_point(D, hq):
    """A sweep point in full on the balanced schedule: every (sequence, head) row."""
    wl = make_config(3, head_dim=D, num_q_heads=hq, kv_format=FP8)
    compare(*run_plan(make_plan(wl, "balanced"), wl, to_dev(wl)), *oracle_full(wl),
            f"fp8 cfg3 D={D} Hq={hq}")


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 257]
EDGE_COMBOS = [  # (block_size, window, sinks, partition)
    (16, 0, False, 0), (16, 0, True, 32), (64, 7, True, 0), (32, 33, False, 64),
    (16, 16, True, 16), (128, 100, False, 128), (256, 1, True, 48),
]


@pytest.mark.parametrize("schedule", ["split", "balanced"])
@pytest.mark.parametrize("combo", range(len(EDGE_COMBOS)))
@pytest.mark.parametrize("D,g", [(D, g) for D in (64, 128, 256) for g in (1, 2, 4, 8)])
def test_fp8_edges(D, g, combo, schedule):
    """Ragged lengths around the 16-token tile, block sizes 16..256, windows, sinks; the
    combination's partition size (unsplit where it is 0), or balanced with 17 workers."""
    bs, W, sinks, P = EDGE_COMBOS[combo]
    wl = make_workload(name="edge", seq_lens=EDGE_LENS, num_q_heads=2 * g, num_kv_heads=2,
                       head_dim=D, block_size=bs, seed=[D, g, combo, 8], window=W,
                       with_sinks=sinks, poison=True, kv_format=FP8, kv_scales=(0.0625, 0.05))
    if schedule == "balanced":
        plan = make_plan(wl, "balanced", num_workers=17)
    else:
        plan = make_plan(wl, "partitioned" if P else "unsplit", partition_size=P)
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"fp8 edge {plan.name} D={D} g={g} bs={bs} W={W} sinks={sinks}")


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_fp8_negative_and_odd_scales(schedule):
    """Scales of either sign, not powers of two: the K scale joins the score scale (its sign
    included) and the V scale multiplies the output."""
    wl = make_workload(name="signs", seq_lens=[300, 17, 1, 1000], num_q_heads=16,
                       num_kv_heads=4, head_dim=128, block_size=16, seed=[21], with_sinks=True,
                       poison=True, kv_format=FP8, kv_scales=(-0.07, -0.0391))
    assert wl.k_scale < 0 and wl.v_scale < 0
    plan = make_plan(wl, schedule, partition_size=64)
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"fp8 negative scales {schedule}")


def test_fp8_graph_replay_balanced():
    """A balanced FP8 step captured in a graph and replayed with new queries written in place:
    every replay equals an eager run bit for bit; the last one also equals the oracle."""
    wl = make_workload(name="context B4 L4096 fp8", seq_lens=[4096] * 4, num_q_heads=32,
                       num_kv_heads=4, head_dim=128, block_size=16, seed=[11, 4, 4096, 8],
                       poison=True, kv_format=FP8, kv_scales=(0.0625, 0.05))
    t = to_dev(wl)
    plan = make_plan(wl, "balanced")
    B, Hq, D = wl.q.shape
    ws = plan.workspace("cuda")
    out = torch.zeros((B, Hq, D), device="cuda")
    lse = torch.zeros((B, Hq), device="cuda")
    args = (t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale))
    kw = dict(k_scale=wl.k_scale, v_scale=wl.v_scale)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(*args, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(*args, out=out, lse=lse, workspace=ws, **kw)
    q0 = t["q"].clone()
    gen = torch.Generator(device="cuda").manual_seed(6)
    for r in range(4):
        t["q"].copy_(torch.randn(q0.shape, device="cuda", generator=gen)
                     .to(torch.bfloat16).view(torch.int16))
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref_out = torch.full_like(out, float("nan"))
        ref_lse = torch.full_like(lse, float("nan"))
        plan.run(*args, out=ref_out, lse=ref_lse, workspace=plan.workspace("cuda"), **kw)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref_out) and torch.equal(got[1], ref_lse), f"replay {r}"
    wl.q[...] = t["q"].cpu().numpy().view(np.uint16)
    compare(got[0].cpu().numpy().astype(np.float64), got[1].cpu().numpy().astype(np.float64),
            *oracle_full(wl), "fp8 graph replay balanced")
    t["q"].copy_(q0)


def test_fp8_default_workers_follow_the_units():
    """A default FP8 plan at head_dim 128 (one query token) takes 8 workers per CU when the batch
    has fewer than four (sequence, KV head) units per CU, and keeps the full count otherwise."""
    import re

    import paged_kv_attention_attn_amd as pa

    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def workers(num_seqs):
        plan = pa.Plan(num_seqs, 32, 8, 4096, 256, 128, 16, schedule="balanced", kv_dtype=FP8)
        return int(re.search(r"_workers(\d+)", plan.name).group(1))

    few = workers(max(1, cus // 4))    # 2 units per CU
    many = workers(max(1, cus // 2))   # 4 units per CU
    log(f"[fp8] default workers: {few} at 2 units per CU, {many} at 4")
    assert few <= 8 * cus
    assert many >= few
    if many > 8 * cus:
        assert few == 8 * cus

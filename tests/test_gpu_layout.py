"""GPU parity for KV pools in other layouts, given to a plan as (block, head, token) strides:
token-major [NB][bs][Hkv][D], K and V interleaved per block [NB][2][Hkv][bs][D], and padded rows
whose padding holds NaN.  The oracle reads the same values from the default layout, so every
schedule (the query-block one included), both KV formats and several query tokens must match it
exactly as before."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from workloads import make_config, make_workload

from gpu_helpers import compare, log, max_len, oracle_full, run_plan, to_dev

pytestmark = pytest.mark.gpu

LAYOUTS = ["token_major", "interleaved", "padded"]


def relayout(wl, t, layout):
    """Device K/V tensors of the workload in `layout`, and the plan's strides (elements)."""
    k, v = wl.k_cache, wl.v_cache               # [NB][Hkv][bs][D], raw bits or codes
    NB, H, bs, D = k.shape
    code = np.uint8 if wl.kv_format == "fp8_e4m3" else np.int16
    dev = torch.device("cuda")
    if layout == "token_major":
        kd = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)).view(code)).to(dev)
        vd = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)).view(code)).to(dev)
        strides = (bs * H * D, D, H * D)
    elif layout == "interleaved":
        buf = torch.from_numpy(np.ascontiguousarray(np.stack([k, v], axis=1)).view(code)).to(dev)
        kd, vd = buf[:, 0], buf[:, 1]            # views: v starts H*bs*D elements after k
        strides = (2 * H * bs * D, bs * D, D)
    else:
        pad = 16 if wl.kv_format == "fp8_e4m3" else 8     # 16 bytes of NaN after every row
        nan = 0x7F if wl.kv_format == "fp8_e4m3" else 0x7FC0
        kp = np.full((NB, H, bs, D + pad), nan, dtype=k.dtype)
        vp = np.full((NB, H, bs, D + pad), nan, dtype=v.dtype)
        kp[..., :D] = k
        vp[..., :D] = v
        kd = torch.from_numpy(kp.view(code)).to(dev)
        vd = torch.from_numpy(vp.view(code)).to(dev)
        strides = (H * bs * (D + pad), bs * (D + pad), D + pad)
    torch.cuda.synchronize()
    return dict(t, k=kd, v=vd), strides


def plan_for(wl, schedule, strides, partition_size=64, num_workers=0):
    return pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule=schedule,
                   partition_size=partition_size, max_seq_len=max_len(wl),
                   num_workers=num_workers, kv_dtype=wl.kv_format, q_len=wl.q_len,
                   kv_layout=strides)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("schedule", ["unsplit", "partitioned", "balanced", "fused"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_layouts_small(layout, schedule, kv):
    wl = make_workload(name="layout", seq_lens=[0, 1, 15, 16, 17, 100, 257, 33], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=32, seed=[3], window=40,
                       with_sinks=True, poison=True, kv_format=kv,
                       kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0))
    t, strides = relayout(wl, to_dev(wl), layout)
    plan = plan_for(wl, schedule, strides, num_workers=7)
    compare(*run_plan(plan, wl, t), *oracle_full(wl), f"{layout} {schedule} {kv}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("D,g", [(64, 8), (128, 1), (256, 4)])
def test_layouts_head_dims_and_groups(D, g, layout):
    wl = make_workload(name="layout", seq_lens=[300, 17, 1, 1000, 64], num_q_heads=2 * g,
                       num_kv_heads=2, head_dim=D, block_size=16, seed=[D, g], poison=True)
    t, strides = relayout(wl, to_dev(wl), layout)
    for schedule in ("balanced", "unsplit"):
        plan = plan_for(wl, schedule, strides)
        compare(*run_plan(plan, wl, t), *oracle_full(wl), f"{layout} D={D} g={g} {schedule}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_layouts_several_query_tokens(layout):
    wl = make_workload(name="layout multi", seq_lens=[0, 2, 17, 100, 257], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, seed=[4], window=20,
                       with_sinks=True, poison=True, q_len=4)
    t, strides = relayout(wl, to_dev(wl), layout)
    plan = plan_for(wl, "balanced", strides, num_workers=9)
    log(f"[layout] {plan.name}")
    compare(*run_plan(plan, wl, t), *oracle_full(wl), f"{layout} q_len=4")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("Q", [4, 40])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_layouts_query_blocks(layout, Q, kv):
    """The query-block schedule reads the pool through the same strides: one wave per block
    (Q = 4: one block of 8 tokens) and workgroups sharing tiles through LDS (Q = 40: 5 blocks),
    whose copies address each 16-byte piece of a row through the row stride."""
    wl = make_workload(name="layout qblock", seq_lens=[0, 2, 17, Q, 100, 257], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=32, seed=[5, Q], window=30,
                       with_sinks=True, poison=True, q_len=Q, kv_format=kv,
                       kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0))
    t, strides = relayout(wl, to_dev(wl), layout)
    plan = plan_for(wl, "query_blocks", strides)
    log(f"[layout] {plan.name}")
    assert ("_w4" in plan.name) == (Q == 40)
    compare(*run_plan(plan, wl, t), *oracle_full(wl), f"{layout} query blocks q_len={Q} {kv}")


def test_token_major_decode_batch_workload():
    """The Llama-8B-shaped step with a token-major pool, against the oracle in full."""
    wl = make_config(2, poison=True)
    t, strides = relayout(wl, to_dev(wl), "token_major")
    compare(*run_plan(plan_for(wl, "balanced", strides), wl, t), *oracle_full(wl),
            "token-major Llama-8B step")


def test_default_strides_equal_no_layout_bitwise():
    wl = make_config(5, seq_lens=[5000, 17, 9000, 4096, 1, 300, 0], poison=True)
    t = to_dev(wl)
    H, bs, D = wl.num_kv_heads, wl.block_size, wl.head_dim
    a = run_plan(plan_for(wl, "balanced", None, num_workers=40), wl, t)
    b = run_plan(plan_for(wl, "balanced", (H * bs * D, bs * D, D), num_workers=40), wl, t)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------------------------
# gather witness of the balanced schedule: the workers' own walk, under every layout
# ---------------------------------------------------------------------------------------------
def check_balanced_witness(wl, t, strides, workers, tag):
    """The rows the balanced walk selects, byte for byte against the oracle's gather from the
    default-layout pool (raw bits or codes), and nothing written past each attended count."""
    from oracle import ref
    from paged_kv_attention_attn_amd import debug

    att = [int(min(L, wl.window)) if wl.window > 0 else int(L) for L in wl.seq_lens]
    max_rows = max(max(att), 1)
    kr, vr = debug.gather_witness_balanced(
        t["k"], t["v"], t["bt"], t["L"], num_seqs=wl.num_seqs, num_kv_heads=wl.num_kv_heads,
        num_blocks=wl.num_blocks, head_dim=wl.head_dim, block_size=wl.block_size,
        num_workers=workers, max_rows=max_rows, window=wl.window, kv_dtype=wl.kv_format,
        kv_layout=strides)
    torch.cuda.synchronize()
    kr, vr = kr.cpu().numpy(), vr.cpu().numpy()
    for b, L in enumerate(wl.seq_lens):
        L = int(L)
        start = max(0, L - wl.window) if wl.window > 0 else 0
        n = L - start
        for kvh in range(wl.num_kv_heads):
            for got, cache in ((kr, wl.k_cache), (vr, wl.v_cache)):
                want = ref.gather_rows(cache, wl.block_table, b, kvh, start, L, wl.block_size)
                want = want.view(np.uint8).reshape(n, got.shape[-1])
                assert np.array_equal(got[b, kvh, :n], want), (tag, b, kvh)
                assert (got[b, kvh, n:] == 0xEE).all(), (tag, b, kvh, "written past the rows")
    log(f"[witness] balanced {tag}: bit-exact over {sum(att) * wl.num_kv_heads} rows")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("layout", ["default"] + LAYOUTS)
@pytest.mark.parametrize("bs,window", [(16, 0), (32, 40), (64, 100)])
def test_balanced_witness_layouts(layout, bs, window, kv):
    wl = make_workload(name="witness", seq_lens=[0, 1, 15, 16, 17, 100, 257, 33, 1000],
                       num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=bs,
                       seed=[bs, window, 5], window=window, poison=True, kv_format=kv,
                       kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0))
    t = to_dev(wl)
    strides = None
    if layout != "default":
        t, strides = relayout(wl, t, layout)
    # one worker, a few, many (units cut between workers), and more than the tiles allow
    for workers in (1, 3, 17, 333, 5000):
        check_balanced_witness(wl, t, strides, workers, f"{layout} bs={bs} W={window} {kv} "
                                                        f"workers={workers}")


@pytest.mark.parametrize("D", [64, 256])
def test_balanced_witness_head_dims(D):
    wl = make_workload(name="witness", seq_lens=[700, 3, 2049, 0, 64], num_q_heads=4,
                       num_kv_heads=4, head_dim=D, block_size=16, seed=[D, 6], window=0,
                       poison=True)
    t, strides = relayout(wl, to_dev(wl), "token_major")
    for workers in (7, 64):
        check_balanced_witness(wl, t, strides, workers, f"D={D} token-major workers={workers}")


def test_balanced_witness_mixed_batch_2048_workers():
    """The first 24 sequences of the mixed batch (window 4096) cut by 2048 workers, about a
    dozen tiles each, default layout."""
    from workloads import config_seq_lens

    wl = make_config(5, seq_lens=config_seq_lens(5)[:24])
    check_balanced_witness(wl, to_dev(wl), None, 2048, "cfg5 first 24 seqs")

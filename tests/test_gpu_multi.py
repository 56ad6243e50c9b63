"""GPU parity of several query tokens per sequence (q_len > 1, causal, token i at position
L - q_len + i) against the fp64 oracle, through paged_attn_plan_run on the balanced schedule:
every (group, q_len) with q_len * group <= 16, every head size, windows, sinks, lengths shorter
than q_len, bf16 and FP8 caches, the decode-batch and mixed workloads (sampled), more tokens
than 16 columns (run in passes), and the argument checks.  The (token, head) pairs of a KV head
are the kernels' columns, so q_len = 1 must equal the one-token plan bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from workloads import make_config, make_workload

from gpu_helpers import (compare, log, make_plan, oracle_full, oracle_multi_triples, run_plan,
                         to_dev)

pytestmark = pytest.mark.gpu

# (group, q_len) with q_len * group <= 16: 16 columns, 8, and padded counts (3, 5 -> 4, 8, 16)
COMBOS = [(1, 2), (1, 3), (1, 5), (1, 8), (1, 16), (2, 2), (2, 3), (2, 5), (2, 8), (4, 2),
          (4, 3), (4, 4), (8, 2)]
EDGE_LENS = [0, 1, 2, 3, 15, 16, 17, 31, 33, 64, 65, 100, 257]


def multi_workload(D, g, Q, *, window=0, sinks=False, kv="bf16", bs=16, lens=EDGE_LENS,
                   seed=0):
    return make_workload(name=f"multi D{D} g{g} Q{Q}", seq_lens=lens, num_q_heads=2 * g,
                         num_kv_heads=2, head_dim=D, block_size=bs,
                         seed=[D, g, Q, window, seed], window=window, with_sinks=sinks,
                         poison=True, kv_format=kv,
                         kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0), q_len=Q)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("g,Q", COMBOS)
def test_multi_edges(g, Q, D, kv):
    wl = multi_workload(D, g, Q, window=0 if (g + Q) % 2 else 7, sinks=(g * Q) % 3 == 0, kv=kv)
    plan = make_plan(wl, "balanced", num_workers=17)
    log(f"[multi] {plan.name}")
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"multi D={D} g={g} Q={Q} kv={kv} W={wl.window} sinks={wl.sinks is not None}")


@pytest.mark.parametrize("workers", [0, 1, 5, 333])
@pytest.mark.parametrize("bs,window", [(16, 0), (64, 33), (32, 1), (256, 100)])
def test_multi_worker_counts_block_sizes_windows(bs, window, workers):
    wl = multi_workload(128, 4, 4, window=window, sinks=True, bs=bs,
                        lens=[300, 17, 1, 1000, 3, 4, 5, 2049], seed=1)
    plan = make_plan(wl, "balanced", num_workers=workers)
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"multi {plan.name} bs={bs} W={window}")


def test_multi_q1_plan_equals_one_token_plan_bitwise():
    wl = make_config(5, seq_lens=[5000, 17, 9000, 4096, 4097, 1, 300, 0], poison=True)
    t = to_dev(wl)
    one = run_plan(make_plan(wl, "balanced", num_workers=50), wl, t)
    plan = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule="balanced",
                   max_seq_len=int(wl.seq_lens.max()), num_workers=50, q_len=1)
    again = run_plan(plan, wl, t)
    assert np.array_equal(one[0], again[0]) and np.array_equal(one[1], again[1])


def sampled(wl, n, seed):
    rng = np.random.default_rng(seed)
    B, Q, Hq = wl.num_seqs, wl.q_len, wl.num_q_heads
    trip = {(int(np.argmax(wl.seq_lens)), Q - 1, 0), (int(np.argmin(wl.seq_lens)), 0, Hq - 1)}
    while len(trip) < n:
        trip.add((int(rng.integers(B)), int(rng.integers(Q)), int(rng.integers(Hq))))
    return sorted(trip)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("Q", [2, 4])
def test_multi_decode_batch_workload(Q, kv):
    """The Llama-8B-shaped batch (B64, 32 q / 8 KV heads: group 4) with Q tokens per sequence:
    sampled (sequence, token, head) triples against the oracle, every output finite."""
    wl = make_config(2, poison=True, kv_format=kv, q_len=Q)
    plan = make_plan(wl, "balanced")
    log(f"[multi] {plan.name}")
    out, lse = run_plan(plan, wl, to_dev(wl))
    trip = sampled(wl, 48, seed=Q)
    eo, el = oracle_multi_triples(wl, trip)
    idx = tuple(np.array(trip).T)
    compare(out[idx], lse[idx], eo, el, f"multi cfg2 Q={Q} kv={kv} ({len(trip)} sampled)")
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_multi_mixed_workload_window_sinks():
    wl = make_config(5, poison=True, q_len=3, seq_lens=[5000, 17, 2, 9000, 4096, 4097, 1, 300])
    out, lse = run_plan(make_plan(wl, "balanced", num_workers=64), wl, to_dev(wl))
    compare(out, lse, *oracle_full(wl), "multi mixed Q=3 window 4096 + sinks")


# 17 to 32 (token, head) pairs: the two-half (32-column) kernels at D <= 128
COMBOS_32 = [(8, 3), (8, 4), (4, 5), (4, 8), (2, 9), (2, 16), (1, 17), (1, 32)]


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("g,Q", COMBOS_32)
def test_multi_32_columns(g, Q, D, kv):
    lens = [0, 1, Q - 1, Q, Q + 1, 17, 100, 257]
    wl = multi_workload(D, g, Q, window=0 if Q % 2 else 9, sinks=g % 2 == 0, kv=kv, lens=lens)
    plan = make_plan(wl, "balanced", num_workers=19)
    log(f"[multi] {plan.name}")
    assert "_c32_" in plan.name and "passes" not in plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"multi 32 columns D={D} g={g} Q={Q} kv={kv} W={wl.window}")


# more (token, head) pairs than one kernel holds (32 at D <= 128, 16 at 256): passes
PASS_COMBOS = [(128, 8, 5), (128, 4, 13), (128, 2, 17), (128, 1, 40), (64, 8, 6),
               (256, 8, 3), (256, 4, 5), (256, 1, 20)]


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D,g,Q", PASS_COMBOS)
def test_multi_in_passes(D, g, Q, kv):
    lens = [0, 1, Q - 1, Q, Q + 1, 17, 100, 257, 1000]
    wl = multi_workload(D, g, Q, window=0 if Q % 2 else 50, sinks=True, kv=kv, lens=lens)
    plan = make_plan(wl, "balanced", num_workers=23)
    log(f"[multi] {plan.name}")
    assert "passes" in plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"multi passes D={D} g={g} Q={Q} kv={kv} W={wl.window}")


def test_multi_plan_rejects_unsupported_requests():
    wl = multi_workload(128, 8, 2)
    with pytest.raises(pa.PagedAttnError):     # above 4096 query tokens
        pa.Plan(2, 16, 2, wl.num_blocks, wl.stride, 128, 16, schedule="balanced", q_len=4097)
    with pytest.raises(pa.PagedAttnError):     # only the balanced schedule takes q_len > 1
        pa.Plan(2, 16, 2, wl.num_blocks, wl.stride, 128, 16, schedule="unsplit", q_len=2)
    with pytest.raises(pa.PagedAttnError):
        pa.Plan(2, 16, 2, wl.num_blocks, wl.stride, 128, 16, schedule="balanced", q_len=0)


def test_multi_graph_replay():
    wl = make_workload(name="multi graph", seq_lens=[4096] * 4, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, block_size=16, seed=[12], poison=True, q_len=4)
    t = to_dev(wl)
    plan = make_plan(wl, "balanced")
    ws = plan.workspace("cuda")
    out = torch.zeros(wl.q.shape, device="cuda")
    lse = torch.zeros(wl.q.shape[:-1], device="cuda")
    args = (t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(*args, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(*args, out=out, lse=lse, workspace=ws)
    gen = torch.Generator(device="cuda").manual_seed(9)
    q0 = t["q"].clone()
    for r in range(3):
        t["q"].copy_(torch.randn(q0.shape, device="cuda", generator=gen)
                     .to(torch.bfloat16).view(torch.int16))
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref_out = torch.full_like(out, float("nan"))
        ref_lse = torch.full_like(lse, float("nan"))
        plan.run(*args, out=ref_out, lse=ref_lse, workspace=plan.workspace("cuda"))
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref_out) and torch.equal(got[1], ref_lse), f"replay {r}"
    wl.q[...] = t["q"].cpu().numpy().view(np.uint16)
    compare(got[0].cpu().numpy().astype(np.float64), got[1].cpu().numpy().astype(np.float64),
            *oracle_full(wl), "multi graph replay")
    t["q"].copy_(q0)


@pytest.mark.parametrize("workers", [7, 50])
def test_multi_nan_key_reaches_only_the_tokens_that_attend_it(workers):
    """Four query tokens per sequence and a NaN in the key at position L - 2 of sequence 1: the
    two tokens before that position do not attend it and stay finite, the two at and after it
    are NaN for that KV head's query heads (units cut into pieces that the fix-up merges)."""
    wl = make_workload(name="multi nan", seq_lens=[200, 90, 333], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[25], poison=True, q_len=4)
    pos = 88
    wl.k_cache[wl.block_table[1, pos // 16], 1, pos % 16, 5] = np.uint16(0x7FC0)
    exp_o, exp_l = oracle_full(wl)
    assert np.isnan(exp_o[1, 2:, 4:8]).all() and not np.isnan(exp_o[1, :2]).any()
    got_o, got_l = run_plan(make_plan(wl, "balanced", num_workers=workers), wl, to_dev(wl))
    bad_o = np.argwhere(np.isnan(got_o) != np.isnan(exp_o))
    assert bad_o.size == 0, f"NaN pattern of out differs at {bad_o[:6].tolist()}"
    assert np.array_equal(np.isnan(got_l), np.isnan(exp_l))
    ok = ~np.isnan(exp_o)
    assert np.abs(got_o[ok] - exp_o[ok]).max() <= 1e-3

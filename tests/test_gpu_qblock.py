"""GPU parity of the query-block schedule (several query tokens per sequence: chunked prefill,
speculative decode) against the fp64 oracle, through paged_attn_plan_run: one wave per
(sequence, KV head, block of 32 / group tokens; 16 / group at head_dim 256), causal tokens at
positions L - q_len + i.  Covered: every head size and group, token counts inside one block and
across many, lengths shorter than q_len (positions below 0) and zero, windows, sinks, block
sizes, bf16 and FP8 caches, XCD-pinned and plain grids, whole-prompt prefill (q_len = L), the
decode-batch workload (sampled), one token, a table entry outside the pool, graph replay, and
the argument checks.  Small batches run with key splits and their merge (plans given a length
bound); the same batches without a bound run unsplit, and the two agree."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from workloads import make_config, make_workload

from gpu_helpers import (compare, log, make_plan, oracle_full, oracle_multi_triples, run_plan,
                         to_dev)

pytestmark = pytest.mark.gpu


def qb_workload(D, g, Q, *, window=0, sinks=False, kv="bf16", bs=16, lens=None, kv_heads=2,
                seed=0):
    if lens is None:
        lens = [0, 1, Q - 1, Q, Q + 1, 17, 100, 257, 1000]
        lens = [max(x, 0) for x in lens]
    return make_workload(name=f"qblock D{D} g{g} Q{Q}", seq_lens=lens, num_q_heads=kv_heads * g,
                         num_kv_heads=kv_heads, head_dim=D, block_size=bs,
                         seed=[D, g, Q, window, seed, 7], window=window, with_sinks=sinks,
                         poison=True, kv_format=kv,
                         kv_scales=(0.0625, 0.05) if kv != "bf16" else (1.0, 1.0), q_len=Q)


# (D, group, q_len): one block, several blocks, a ragged last block, one token per block
COMBOS = [(64, 1, 40), (64, 2, 100), (64, 4, 9), (64, 8, 70), (128, 1, 1), (128, 1, 33),
          (128, 2, 16), (128, 4, 8), (128, 4, 70), (128, 8, 5), (128, 8, 4), (256, 1, 17),
          (256, 2, 40), (256, 4, 9), (256, 8, 6), (256, 8, 2)]


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D,g,Q", COMBOS)
def test_qblock_edges(D, g, Q, kv):
    wl = qb_workload(D, g, Q, window=0 if (g + Q) % 2 else 11, sinks=(g * Q) % 3 == 0, kv=kv)
    plan = make_plan(wl, "query_blocks")
    log(f"[qblock] {plan.name}")
    assert plan.name.startswith("pa_qblock_")
    assert (plan.workspace_size > 0) == ("_s" in plan.name.replace("_xcd", ""))
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"qblock D={D} g={g} Q={Q} kv={kv} W={wl.window} sinks={wl.sinks is not None}")


@pytest.mark.parametrize("bs,window", [(16, 0), (64, 33), (32, 1), (256, 100)])
def test_qblock_block_sizes_windows(bs, window):
    wl = qb_workload(128, 4, 40, window=window, sinks=True, bs=bs,
                     lens=[300, 17, 1, 1000, 3, 40, 41, 2049], seed=1)
    plan = make_plan(wl, "query_blocks")
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"qblock {plan.name} bs={bs} W={window}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_qblock_xcd_pinned_grid(kv):
    """8 sequences x 2 KV heads = 16 units, a multiple of the 8 XCDs: every block of a unit on
    one XCD."""
    wl = qb_workload(128, 4, 50, window=0, sinks=False, kv=kv,
                     lens=[50, 60, 1, 0, 500, 49, 51, 1300], seed=2)
    plan = make_plan(wl, "query_blocks")
    log(f"[qblock] {plan.name}")
    assert plan.name.endswith("_xcd")
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"qblock xcd-pinned kv={kv}")


@pytest.mark.parametrize("D,g", [(128, 4), (128, 8), (64, 1), (256, 8)])
def test_qblock_whole_prompt_prefill(D, g):
    """Every token of every sequence is new (q_len = L): plain causal self-attention."""
    Q = 300
    wl = qb_workload(D, g, Q, lens=[Q] * 4, kv_heads=2, seed=3)
    plan = make_plan(wl, "query_blocks")
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"qblock prefill D={D} g={g}")


def sampled(wl, n, seed):
    rng = np.random.default_rng(seed)
    B, Q, Hq = wl.num_seqs, wl.q_len, wl.num_q_heads
    trip = {(int(np.argmax(wl.seq_lens)), Q - 1, 0), (int(np.argmin(wl.seq_lens)), 0, Hq - 1)}
    while len(trip) < n:
        trip.add((int(rng.integers(B)), int(rng.integers(Q)), int(rng.integers(Hq))))
    return sorted(trip)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_qblock_decode_batch_workload(kv):
    """The Llama-8B-shaped batch (B64, 32 q / 8 KV heads) with 64 new tokens per sequence:
    sampled (sequence, token, head) triples against the oracle, every output finite."""
    wl = make_config(2, poison=True, kv_format=kv, q_len=64)
    plan = make_plan(wl, "query_blocks")
    log(f"[qblock] {plan.name}")
    out, lse = run_plan(plan, wl, to_dev(wl))
    trip = sampled(wl, 48, seed=11)
    eo, el = oracle_multi_triples(wl, trip)
    idx = tuple(np.array(trip).T)
    compare(out[idx], lse[idx], eo, el, f"qblock cfg2 Q=64 kv={kv} ({len(trip)} sampled)")
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_qblock_mixed_workload_window_sinks():
    wl = make_config(5, poison=True, q_len=9, seq_lens=[5000, 17, 2, 9000, 4096, 4097, 1, 300])
    out, lse = run_plan(make_plan(wl, "query_blocks"), wl, to_dev(wl))
    compare(out, lse, *oracle_full(wl), "qblock mixed Q=9 window 4096 + sinks")


def test_qblock_bad_table_entry_gives_nan_for_that_sequence_only():
    wl = qb_workload(128, 4, 20, lens=[200, 150, 90], seed=4)
    t = to_dev(wl)
    bt = t["bt"].clone()
    bt[1, 3] = wl.num_blocks          # outside the pool, inside sequence 1's attended range
    t["bt"] = bt
    out, lse = run_plan(make_plan(wl, "query_blocks"), wl, t)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    eo, el = oracle_full(wl)
    keep = [0, 2]
    compare(out[keep], lse[keep], eo[keep], el[keep], "qblock sequences with good tables")


def test_qblock_key_splits_bad_table_entry_and_length():
    """A plan with key splits: a table entry outside the pool in a middle split of sequence 0,
    and a length above what sequence 2's table row holds.  Both sequences come out NaN (their
    splits' NaN LSEs travel through the merge); sequence 1 matches the oracle."""
    wl = qb_workload(128, 4, 20, lens=[4000, 150, 3000], seed=12)
    t = to_dev(wl)
    plan = make_plan(wl, "query_blocks")
    log(f"[qblock] {plan.name}")
    splits = int(plan.name.split("_s")[-1].split("_")[0])
    assert splits >= 8, plan.name
    bt = t["bt"].clone()
    bt[0, 120] = wl.num_blocks        # tile 120 of 250: a middle split of sequence 0
    L = t["L"].clone()
    L[2] = wl.stride * wl.block_size + 5
    t["bt"], t["L"] = bt, L
    out, lse = run_plan(plan, wl, t)
    for b in (0, 2):
        assert np.isnan(out[b]).all() and np.isnan(lse[b]).all(), b
    eo, el = oracle_full(wl)
    compare(out[[1]], lse[[1]], eo[[1]], el[[1]], "qblock split plan, the good sequence")


def test_qblock_graph_replay_matches_eager():
    wl = qb_workload(128, 4, 33, window=200, sinks=True, lens=[100, 33, 500, 7], seed=5)
    t = to_dev(wl)
    plan = make_plan(wl, "query_blocks")
    assert "_s" in plan.name   # key splits and their merge, captured together
    ws = plan.workspace("cuda")
    args = (t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale))
    out = torch.empty(wl.q.shape, device="cuda")
    lse = torch.empty(wl.q.shape[:-1], device="cuda")
    plan.run(*args, out=out, lse=lse, sinks=t["sinks"], workspace=ws)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan.run(*args, out=out, lse=lse, sinks=t["sinks"], workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    compare(ref_out.cpu().numpy().astype(np.float64), ref_lse.cpu().numpy().astype(np.float64),
            *oracle_full(wl), "qblock eager (graph reference)")


def test_qblock_plan_rejects_unsupported_requests():
    wl = qb_workload(128, 4, 2, lens=[10, 20])
    with pytest.raises(pa.PagedAttnError):     # 16 heads per KV head: no kernel
        pa.Plan(2, 32, 2, wl.num_blocks, wl.stride, 128, 16, schedule="query_blocks", q_len=2)
    with pytest.raises(pa.PagedAttnError):
        pa.Plan(2, 8, 2, wl.num_blocks, wl.stride, 128, 16, schedule="query_blocks", q_len=0)
    with pytest.raises(pa.PagedAttnError):
        pa.Plan(2, 8, 2, wl.num_blocks, wl.stride, 128, 16, schedule="query_blocks", q_len=4097)


def plan_without_bound(wl):
    """A query-block plan with no length bound: never key splits."""
    return pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule="query_blocks",
                   max_seq_len=0, kv_dtype=wl.kv_format, q_len=wl.q_len)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("D,g,Q", [(64, 2, 100), (128, 4, 70), (128, 8, 5), (256, 4, 9),
                                   (256, 8, 2)])
def test_qblock_with_and_without_key_splits(D, g, Q, kv):
    """The same small batch with and without key splits: both against the oracle, and within
    fp32 rounding of each other."""
    wl = qb_workload(D, g, Q, window=0 if Q % 2 else 1500, sinks=True, kv=kv,
                     lens=[0, 1, Q, Q + 1, 300, 1000, 4100], seed=9)
    t = to_dev(wl)
    split = make_plan(wl, "query_blocks")
    whole = plan_without_bound(wl)
    log(f"[qblock] {split.name} / {whole.name}")
    assert "_s" in split.name and whole.workspace_size == 0
    assert "_s" not in whole.name.replace("_xcd", "")
    a = run_plan(split, wl, t)
    b = run_plan(whole, wl, t)
    ref = oracle_full(wl)
    compare(*a, *ref, f"qblock split D={D} g={g} Q={Q} kv={kv}")
    compare(*b, *ref, f"qblock whole D={D} g={g} Q={Q} kv={kv}")
    fin = np.isfinite(a[1])
    assert np.array_equal(fin, np.isfinite(b[1]))
    assert np.abs(a[0] - b[0]).max() <= 1e-4 and np.abs(a[1][fin] - b[1][fin]).max() <= 1e-4


def test_qblock_key_splits_with_lengths_above_the_bound():
    """Lengths above the plan's bound: the last split takes the rest of the keys."""
    wl = qb_workload(128, 4, 40, sinks=True, lens=[50, 3000, 700, 41], seed=10)
    t = to_dev(wl)
    plan = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, schedule="query_blocks", max_seq_len=512,
                   q_len=wl.q_len)
    log(f"[qblock] {plan.name}")
    assert "_s" in plan.name
    compare(*run_plan(plan, wl, t), *oracle_full(wl), "qblock lengths above the bound")


@pytest.mark.parametrize("D,g,Q,lens,window", [
    (128, 4, 300, [300] * 4, 0),                    # whole prompts: the rows with fewest keys
    (128, 4, 70, None, 11),                         # edge lengths, a window
    (64, 2, 100, None, 0),
    (128, 8, 64, [64, 2000, 700, 5], 0),
    (64, 8, 40, [40, 41, 1000, 3], 300),
])
def test_qblock_one_term_p(D, g, Q, lens, window):
    """Plans with p_terms=1 (PA_PLAN_P_ONE_BF16): P rounded to one bf16 term in the 32-key form.
    |p~ - p| <= 2^-8 p and the denominator keeps fp32 p, so an output moves by at most 2^-8
    max|v| from the two-term result (which meets the 1e-3 gate); the LSE does not move.  Both
    bounds hold against the oracle, inside the 3e-2 contract."""
    wl = qb_workload(D, g, Q, lens=lens, window=window, sinks=True, seed=11)
    t = to_dev(wl)
    one = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                  wl.head_dim, wl.block_size, window=wl.window, schedule="query_blocks",
                  q_len=wl.q_len, p_terms=1)
    two = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                  wl.head_dim, wl.block_size, window=wl.window, schedule="query_blocks",
                  q_len=wl.q_len)
    log(f"[qblock] {one.name} / {two.name}")
    assert one.name == two.name + "_p1"
    v = (wl.v_cache.astype(np.uint32) << 16).view(np.float32)
    vmax = float(np.abs(v[np.isfinite(v)]).max())
    bound = 2.0 ** -8 * vmax
    ref = oracle_full(wl)
    a = run_plan(one, wl, t)
    b = run_plan(two, wl, t)
    stats = compare(*a, *ref, f"qblock one-term P D={D} g={g} Q={Q}", strict=False)
    compare(*b, *ref, f"qblock two-term P D={D} g={g} Q={Q}")
    assert stats["max_abs"] <= bound + 1e-3, (stats, bound)
    assert stats["lse_max_abs"] <= 1e-3, stats
    assert np.abs(a[0] - b[0]).max() <= bound + 1e-5
    fin = np.isfinite(b[1])
    assert np.array_equal(fin, np.isfinite(a[1]))
    assert np.abs(a[1][fin] - b[1][fin]).max() <= 1e-5


def test_qblock_one_term_p_key_splits_graph_replay():
    """One bf16 term of P with key splits (a small batch and a length bound) and their merge,
    captured in a graph: every replay bit-equal to the eager run, which holds the one-term bound
    against the oracle."""
    wl = qb_workload(128, 4, 33, window=200, sinks=True, lens=[100, 33, 500, 7], seed=12)
    t = to_dev(wl)
    plan = pa.Plan(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.stride,
                   wl.head_dim, wl.block_size, window=wl.window, schedule="query_blocks",
                   max_seq_len=int(wl.seq_lens.max()), q_len=wl.q_len, p_terms=1)
    log(f"[qblock] {plan.name}")
    assert "_s" in plan.name and plan.name.endswith("_p1")
    ws = plan.workspace("cuda")
    args = (t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale))
    out = torch.empty(wl.q.shape, device="cuda")
    lse = torch.empty(wl.q.shape[:-1], device="cuda")
    plan.run(*args, out=out, lse=lse, sinks=t["sinks"], workspace=ws)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan.run(*args, out=out, lse=lse, sinks=t["sinks"], workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    v = (wl.v_cache.astype(np.uint32) << 16).view(np.float32)
    bound = 2.0 ** -8 * float(np.abs(v[np.isfinite(v)]).max())
    stats = compare(ref_out.cpu().numpy().astype(np.float64),
                    ref_lse.cpu().numpy().astype(np.float64), *oracle_full(wl),
                    "qblock one-term P, key splits (graph reference)", strict=False)
    assert stats["max_abs"] <= bound + 1e-3 and stats["lse_max_abs"] <= 1e-3, (stats, bound)

"""GPU tests of the KV-head-pair balanced kernels: a prepared balanced plan with one query token
(bf16 or FP8 KV), an even number of KV heads and 2 or 4 query heads per KV head streams two
adjacent KV heads per unit.  Parity with the fp64 oracle over the edge lengths, block sizes, windows, sinks
and worker counts; NaN isolation between the two heads of a pair; plans that must not pair."""
from __future__ import annotations

import numpy as np
import pytest

from workloads import FP8_QNAN, make_config, make_workload

from gpu_helpers import compare, log, make_plan, oracle_full, run_plan, to_dev

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 257]
EDGE_COMBOS = [  # (block_size, window, sinks)
    (16, 0, False), (16, 0, True), (64, 7, True), (32, 33, False), (16, 16, True),
    (128, 100, False), (256, 1, True),
]


def pairs_expected(wl) -> bool:
    """The plans that pair KV heads: one query token, an even number of KV heads, 2 or 4 query
    heads per KV head, head_dim 64."""
    g = wl.num_q_heads // wl.num_kv_heads
    return wl.q_len == 1 and wl.num_kv_heads % 2 == 0 and g in (2, 4) and wl.head_dim == 64


def scales(kv):
    return (0.0625, 0.05) if kv != "bf16" else (1.0, 1.0)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("workers", [0, 3, 17])
@pytest.mark.parametrize("combo", range(len(EDGE_COMBOS)))
@pytest.mark.parametrize("D,g,hkv", [(64, 2, 2), (64, 4, 4), (128, 2, 4), (128, 4, 2),
                                     (128, 4, 6)])
def test_pair_edges(D, g, hkv, combo, workers, kv):
    bs, W, sinks = EDGE_COMBOS[combo]
    wl = make_workload(name="pair edge", seq_lens=EDGE_LENS, num_q_heads=hkv * g,
                       num_kv_heads=hkv, head_dim=D, block_size=bs, seed=[D, g, hkv, combo, 3],
                       window=W, with_sinks=sinks, poison=True, kv_format=kv,
                       kv_scales=scales(kv))
    plan = make_plan(wl, "balanced", num_workers=workers)
    assert ("headpairs" in plan.name) == pairs_expected(wl), plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"pairs {kv} D={D} g={g} Hkv={hkv} bs={bs} W={W} sinks={sinks} workers={workers}")


@pytest.mark.parametrize("D,g,hkv,kv", [(128, 4, 3, "fp8_e4m3"), (64, 8, 2, "bf16"),
                                        (64, 1, 4, "bf16"), (256, 4, 2, "fp8_e4m3"),
                                        (128, 4, 2, "bf16")])
def test_plans_that_do_not_pair(D, g, hkv, kv):
    wl = make_workload(name="no pair", seq_lens=EDGE_LENS, num_q_heads=hkv * g,
                       num_kv_heads=hkv, head_dim=D, block_size=16, seed=[D, g, hkv, 4],
                       with_sinks=True, poison=True, kv_format=kv, kv_scales=scales(kv))
    plan = make_plan(wl, "balanced")
    assert not pairs_expected(wl) and "headpairs" not in plan.name, plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"no pairs D={D} g={g}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("workers", [0, 1024, 4096])
def test_pair_sweep_point_in_full(workers, kv):
    """The head_dim-64 sweep point (B32, L 8192, 32 query / 8 KV heads), poisoned, in full."""
    wl = make_config(3, head_dim=64, num_q_heads=32, poison=True, kv_format=kv)
    plan = make_plan(wl, "balanced", num_workers=workers)
    log(f"[pairs] {plan.name}")
    assert "headpairs" in plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl),
            f"pairs {kv} sweep D64 hq32 workers={workers}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_pair_mixed_batch_at_head_dim_64(kv):
    """The mixed batch's lengths, window 4096 and sinks, at head_dim 64 (8 KV heads of 4),
    poisoned, in full."""
    from workloads import config_seq_lens
    wl = make_workload(name="mixed D64", seq_lens=config_seq_lens(5), num_q_heads=32,
                       num_kv_heads=8, head_dim=64, block_size=16, seed=[26], window=4096,
                       with_sinks=True, poison=True, kv_format=kv, kv_scales=scales(kv))
    plan = make_plan(wl, "balanced", num_workers=333)
    assert "headpairs" in plan.name
    compare(*run_plan(plan, wl, to_dev(wl)), *oracle_full(wl), f"pairs {kv} mixed D64")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("head", [0, 1])
def test_nan_stays_in_its_head(which, head, kv):
    """A NaN in an attended K or V row of one head of a pair reaches only that head's query
    heads (K: all their outputs; V: the one dimension), never the other head's."""
    D = 64
    wl = make_workload(name="pair nan", seq_lens=[200, 90, 333], num_q_heads=8, num_kv_heads=2,
                       head_dim=D, block_size=16, seed=[23], poison=True, kv_format=kv,
                       kv_scales=scales(kv))
    cache = wl.k_cache if which == "k" else wl.v_cache
    tok = 77
    cache[wl.block_table[1, tok // 16], head, tok % 16, 5] = \
        FP8_QNAN if kv != "bf16" else np.uint16(0x7FC0)
    exp_o, exp_l = oracle_full(wl)
    heads = slice(4 * head, 4 * head + 4)
    assert np.isnan(exp_o[1, heads, 5]).all()
    plan = make_plan(wl, "balanced", num_workers=7)
    assert "headpairs" in plan.name
    got_o, got_l = run_plan(plan, wl, to_dev(wl))
    bad_o = np.argwhere(np.isnan(got_o) != np.isnan(exp_o))
    bad_l = np.argwhere(np.isnan(got_l) != np.isnan(exp_l))
    assert bad_o.size == 0, f"NaN pattern of out differs at {bad_o[:6].tolist()} " \
        f"({len(bad_o)} places; got {int(np.isnan(got_o).sum())} NaN, want " \
        f"{int(np.isnan(exp_o).sum())})"
    assert bad_l.size == 0, f"NaN pattern of lse differs at {bad_l[:6].tolist()}"
    ok = ~np.isnan(exp_o)
    assert np.abs(got_o[ok] - exp_o[ok]).max() <= 1e-3


def test_pairs_equal_single_heads_at_length_one():
    """L = 1 is order-free: the pair kernel returns each head's V row bit for bit."""
    wl = make_workload(name="pair L1", seq_lens=[1] * 9, num_q_heads=16, num_kv_heads=4,
                       head_dim=64, block_size=16, seed=[24], poison=True)
    plan = make_plan(wl, "balanced", num_workers=5)
    assert "headpairs" in plan.name
    out, _ = run_plan(plan, wl, to_dev(wl))
    exp, _ = oracle_full(wl)
    assert np.array_equal(out, exp)

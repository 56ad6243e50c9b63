"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded bf16
inputs.  Contract: max abs error <= 3e-2 on out and lse; the tests also hold the far tighter
regression gates of gpu_helpers (fp32 accumulation lands ~1e-6 from fp64).  Integer work (the
block-table walk) is checked bit-exactly through the gather witness."""
import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from paged_kv_attention_attn_amd import debug
from oracle import ref
from workloads import SWEEP_POINTS, config_seq_lens, make_config, make_workload

from gpu_helpers import (BALANCED, bench_partition, compare, log, max_len, oracle_full, run_gpu,
                         to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_present():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    name = torch.cuda.get_device_properties(0).gcnArchName
    log(f"[gpu] {torch.cuda.get_device_name(0)} {name}")
    assert name.startswith("gfx950"), name


@pytest.fixture(params=["mfma_pv", "mfma", "valu"])
def qk_path(request, monkeypatch):
    """Run the test on every score path: q.k and P.V on the matrix cores, q.k on the matrix
    cores with P.V on the vector ALUs, both on the vector ALUs."""
    monkeypatch.setenv("PA_DECODE_PATH", request.param)
    return request.param


def f32_of_bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------------------------
def test_config1_unsplit(qk_path):
    wl = make_config(1)
    t = to_dev(wl)
    compare(*run_gpu(wl, t), *oracle_full(wl), f"cfg1 unsplit {qk_path}")


@pytest.mark.parametrize("P", [16, 32, 48, 64, 112])
def test_config1_split(P, qk_path):
    wl = make_config(1)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=P), *oracle_full(wl), f"cfg1 split P={P} {qk_path}")


@pytest.mark.parametrize("P", [0, 32])
def test_config1_poisoned(P, qk_path):
    wl = make_config(1, poison=True)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=P), *oracle_full(wl),
            f"cfg1 poisoned P={P} {qk_path}")


def test_config2_bench_launch():
    wl = make_config(2)
    t = to_dev(wl)
    P = bench_partition(wl)
    exp = oracle_full(wl)
    compare(*run_gpu(wl, t, partition_size=P), *exp, f"cfg2 split P={P}")
    compare(*run_gpu(wl, t), *exp, "cfg2 unsplit")


def test_config2_both_paths_and_wave_counts(monkeypatch):
    wl = make_config(2)
    t = to_dev(wl)
    exp = oracle_full(wl)
    for path in ("valu", "mfma", "mfma_pv"):
        for waves in ("1", "2", "4", "8"):
            monkeypatch.setenv("PA_DECODE_PATH", path)
            monkeypatch.setenv("PA_DECODE_WAVES", waves)
            compare(*run_gpu(wl, t, partition_size=1024), *exp,
                    f"cfg2 {path} waves={waves} P=1024")


def test_config2_poisoned():
    wl = make_config(2, poison=True)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=bench_partition(wl)), *oracle_full(wl),
            "cfg2 poisoned")


@pytest.mark.parametrize("D,hq", SWEEP_POINTS)
def test_config3_point(D, hq):
    """A sweep point in full: every (sequence, head) row of the fixed-partition schedule (the
    library's suggested partition size) and of the balanced schedule against the whole-batch
    oracle."""
    wl = make_config(3, head_dim=D, num_q_heads=hq)
    t = to_dev(wl)
    exp = oracle_full(wl)
    P = bench_partition(wl)
    compare(*run_gpu(wl, t, partition_size=P), *exp, f"cfg3 D={D} Hq={hq} P={P}")
    compare(*run_gpu(wl, t, partition_size=BALANCED), *exp, f"cfg3 balanced D={D} Hq={hq}")


def test_config4_long_context():
    wl = make_config(4)
    t = to_dev(wl)
    out, lse = run_gpu(wl, t, partition_size=512)
    compare(out, lse, *oracle_full(wl), "cfg4 split P=512")


def test_config5_window_sinks():
    wl = make_config(5)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_gpu(wl, t), *exp, "cfg5 unsplit")
    compare(*run_gpu(wl, t, partition_size=bench_partition(wl)), *exp, "cfg5 split")


def test_config5_poisoned():
    wl = make_config(5, poison=True)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_gpu(wl, t), *exp, "cfg5 poisoned unsplit")
    compare(*run_gpu(wl, t, partition_size=512), *exp, "cfg5 poisoned split")


# ---------------------------------------------------------------------------------------------
# small cases spanning several tiles and ragged tails, every head size and group
# ---------------------------------------------------------------------------------------------
EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 257]
EDGE_COMBOS = [  # (block_size, window, sinks, partition)
    (16, 0, False, 0), (16, 0, True, 32), (64, 7, True, 0), (32, 33, False, 64),
    (16, 16, True, 16), (128, 100, False, 128), (256, 1, True, 48),
]


@pytest.mark.parametrize("combo", range(len(EDGE_COMBOS)))
@pytest.mark.parametrize("D,g", [(D, g) for D in (64, 128, 256) for g in (1, 2, 4, 8)])
def test_edges(D, g, combo, qk_path):
    bs, W, sinks, P = EDGE_COMBOS[combo]
    wl = make_workload(name="edge", seq_lens=EDGE_LENS, num_q_heads=2 * g, num_kv_heads=2,
                       head_dim=D, block_size=bs, seed=[D, g, combo], window=W,
                       with_sinks=sinks, poison=True)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=P), *oracle_full(wl),
            f"edge {qk_path} D={D} g={g} bs={bs} W={W} sinks={sinks} P={P}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_seq_len_one_is_v_row_bit_exact(D, qk_path):
    wl = make_workload(name="L1", seq_lens=[1, 1, 1, 1], num_q_heads=8, num_kv_heads=2,
                       head_dim=D, block_size=16, seed=[1, D], poison=True)
    t = to_dev(wl)
    for P in (0, 16):
        out, _ = run_gpu(wl, t, partition_size=P)
        for b in range(4):
            phys = wl.block_table[b, 0]
            for h in range(8):
                vrow = f32_of_bf16(wl.v_cache[phys, h // 4, 0]).astype(np.float64)
                assert np.array_equal(out[b, h], vrow), (P, b, h)


def test_block_permutation_invariance_bitwise():
    wl = make_config(2, seq_lens=[700, 33, 1500, 16, 2049, 1])
    t = to_dev(wl)
    base = run_gpu(wl, t, partition_size=256)
    sigma = np.random.default_rng(9).permutation(wl.num_blocks)
    k2 = np.empty_like(wl.k_cache)
    v2 = np.empty_like(wl.v_cache)
    k2[sigma] = wl.k_cache
    v2[sigma] = wl.v_cache
    wl.k_cache, wl.v_cache = k2, v2
    wl.block_table = sigma[wl.block_table].astype(np.int32)
    t2 = to_dev(wl)
    again = run_gpu(wl, t2, partition_size=256)
    assert np.array_equal(base[0], again[0]) and np.array_equal(base[1], again[1])


def test_repeat_runs_are_bit_identical():
    wl = make_config(5, seq_lens=[5000, 17, 9000, 4096, 4097, 1, 300])
    t = to_dev(wl)
    a = run_gpu(wl, t, partition_size=512)
    for _ in range(3):
        b = run_gpu(wl, t, partition_size=512)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lse_null_leaves_neighbours_untouched():
    wl = make_config(1)
    t = to_dev(wl)
    B, Hq, D = wl.q.shape
    n = B * Hq * D
    buf = torch.full((n + 4096,), 12345.0, device="cuda")
    out = buf[:n].view(B, Hq, D)
    pa.decode(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale), out=out, lse=None,
              want_lse=False)
    torch.cuda.synchronize()
    assert bool((buf[n:] == 12345.0).all())
    eo, _ = oracle_full(wl)
    assert np.abs(out.cpu().numpy() - eo).max() < 1e-3


def test_unused_table_entries_may_hold_anything(qk_path):
    wl = make_workload(name="inv", seq_lens=[3, 40, 17, 0, 64], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[4], stride=12, unused_entry="invalid",
                       poison=True)
    assert (wl.block_table == -1).any()
    t = to_dev(wl)
    for P in (0, 16, 32):
        compare(*run_gpu(wl, t, partition_size=P), *oracle_full(wl), f"-1 unused entries P={P}")


def test_bad_table_entry_poisons_only_its_sequence(qk_path):
    wl = make_workload(name="bad", seq_lens=[40, 40, 40], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[5])
    exp = oracle_full(wl)
    wl.block_table[1, 1] = wl.num_blocks          # out of range, attended
    wl.block_table[2, 0] = -7                     # negative, attended
    t = to_dev(wl)
    for P in (0, 16):
        out, lse = run_gpu(wl, t, partition_size=P)
        assert np.isnan(out[1]).all() and np.isnan(out[2]).all() and np.isnan(lse[1:]).all()
        assert np.abs(out[0] - exp[0][0]).max() < 1e-3


def test_length_beyond_table_or_partitions_is_nan(qk_path):
    wl = make_workload(name="len", seq_lens=[40, 40], num_q_heads=4, num_kv_heads=2,
                       head_dim=64, block_size=16, seed=[6])
    exp = oracle_full(wl)
    t = to_dev(wl)
    t["L"] = torch.tensor([40, 49], dtype=torch.int32, device="cuda")    # stride 3 * 16 = 48
    out, lse = run_gpu(wl, t)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    assert np.abs(out[0] - exp[0][0]).max() < 1e-3
    t["L"] = torch.tensor([32, 33], dtype=torch.int32, device="cuda")    # 33 needs 3 of P=16
    out, lse = run_gpu(wl, t, partition_size=16, max_partitions=2)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    for h in range(4):
        eo, _ = ref.decode_one(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                               np.array([32, 33], np.int32), wl.scale, 16, 0, h)
        assert np.abs(out[0, h] - eo).max() < 1e-3


# ---------------------------------------------------------------------------------------------
# gather witness: the decode kernels' address generator, bit-exact against the oracle gather
# ---------------------------------------------------------------------------------------------
def check_witness(wl, tag):
    t = to_dev(wl)
    W = wl.window
    attended = [min(int(L), W) if W > 0 else int(L) for L in wl.seq_lens]
    rows = max(1, max(attended))
    kr, vr = debug.gather_witness(t["k"], t["v"], t["bt"], t["L"], num_seqs=wl.num_seqs,
                                  window=W, max_rows=rows)
    torch.cuda.synchronize()
    kr = kr.cpu().numpy().view(np.uint16)
    vr = vr.cpu().numpy().view(np.uint16)
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        start, stop = ref.attended_range(L, W)
        n = stop - start
        for kvh in range(wl.num_kv_heads):
            ek = ref.gather_rows(wl.k_cache, wl.block_table, b, kvh, start, stop, wl.block_size)
            ev = ref.gather_rows(wl.v_cache, wl.block_table, b, kvh, start, stop, wl.block_size)
            assert np.array_equal(kr[b, kvh, :n], ek), (tag, b, kvh)
            assert np.array_equal(vr[b, kvh, :n], ev), (tag, b, kvh)
            assert (kr[b, kvh, n:] == 0xFFFF).all() and (vr[b, kvh, n:] == 0xFFFF).all()
    log(f"[witness] {tag}: bit-exact over {sum(attended) * wl.num_kv_heads} rows")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("bs,W", [(16, 0), (64, 0), (16, 37), (32, 100), (256, 5)])
def test_witness_small(D, bs, W):
    wl = make_workload(name="wit", seq_lens=EDGE_LENS, num_q_heads=4, num_kv_heads=2,
                       head_dim=D, block_size=bs, seed=[D, bs, W], window=W)
    check_witness(wl, f"D={D} bs={bs} W={W}")


def test_witness_config2_and_5():
    check_witness(make_config(2, seq_lens=config_seq_lens(2)[:16]), "cfg2 first 16 seqs")
    check_witness(make_config(5, seq_lens=config_seq_lens(5)[:24]), "cfg5 first 24 seqs")


# ---------------------------------------------------------------------------------------------
# split partials and the reduce kernel on their own
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("P,W,sinks", [(32, 0, True), (64, 45, True), (16, 0, False)])
def test_partials_match_oracle_partitions(P, W, sinks, qk_path):
    wl = make_workload(name="part", seq_lens=EDGE_LENS, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[P, W], window=W, with_sinks=sinks,
                       poison=True)
    t = to_dev(wl)
    pmax = pa.num_partitions(max_len(wl), P)
    part, plse = pa.decode(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale), window=W,
                           sinks=t["sinks"], partition_size=P, max_partitions=pmax)
    torch.cuda.synchronize()
    eo, el = ref.decode_partitions(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                   wl.scale, wl.block_size, P, max_partitions=pmax, window=W,
                                   sinks=wl.sinks)
    part = part.cpu().numpy().astype(np.float64)
    plse = plse.cpu().numpy().astype(np.float64)
    for b, L in enumerate(wl.seq_lens):
        n = pa.num_partitions(int(L), P)
        compare(part[b, :, :n].reshape(-1, 128), plse[b, :, :n].reshape(-1),
                eo[b, :, :n].reshape(-1, 128), el[b, :, :n].reshape(-1), f"partials b={b}")


def test_reduce_kernel_on_oracle_partials():
    rng = np.random.default_rng(12)
    B, Hq, Pmax, D, P = 5, 6, 9, 128, 64
    L = np.array([0, 1, 64, 65, 9 * 64], np.int32)
    o = rng.standard_normal((B, Hq, Pmax, D)).astype(np.float32)
    l = (rng.standard_normal((B, Hq, Pmax)) * 3).astype(np.float32)
    # empty partitions: lse = -inf and a NaN row that must never be read
    l[1, :, 0] = -np.inf
    o[1, :, 0] = np.nan
    l[3, 2, 1] = -np.inf
    o[3, 2, 1] = np.nan
    l[0, :, 0] = -np.inf
    counts = np.array([pa.num_partitions(int(x), P) for x in L])
    eo, el = ref.merge_partitions(o.astype(np.float64), l.astype(np.float64), counts)
    dev = torch.device("cuda")
    out, lse = pa.reduce(torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev),
                         torch.from_numpy(L).to(dev), partition_size=P)
    torch.cuda.synchronize()
    compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), eo, el,
            "reduce on oracle partials")


# ---------------------------------------------------------------------------------------------
# balanced schedule (persistent workers, fix-up merge)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("workers", [0, 1, 2, 3, 5, 64])
def test_config1_balanced(workers, qk_path):
    wl = make_config(1, poison=True)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=BALANCED, num_workers=workers), *oracle_full(wl),
            f"cfg1 balanced workers={workers} {qk_path}")


@pytest.mark.parametrize("workers", [0, 7, 1000])
def test_config2_balanced(workers):
    wl = make_config(2)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=BALANCED, num_workers=workers), *oracle_full(wl),
            f"cfg2 balanced workers={workers}")


def test_config2_balanced_valu_and_poisoned(monkeypatch):
    wl = make_config(2, poison=True)
    t = to_dev(wl)
    exp = oracle_full(wl)
    compare(*run_gpu(wl, t, partition_size=BALANCED), *exp, "cfg2 balanced poisoned default")
    for path in ("mfma", "valu"):
        monkeypatch.setenv("PA_DECODE_PATH", path)
        compare(*run_gpu(wl, t, partition_size=BALANCED), *exp, f"cfg2 balanced poisoned {path}")


def test_config4_balanced():
    wl = make_config(4)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=BALANCED), *oracle_full(wl), "cfg4 balanced")


def test_config5_balanced():
    wl = make_config(5, poison=True)
    t = to_dev(wl)
    exp = oracle_full(wl)
    for workers in (0, 333):
        compare(*run_gpu(wl, t, partition_size=BALANCED, num_workers=workers), *exp,
                f"cfg5 balanced poisoned workers={workers}")


@pytest.mark.parametrize("workers", [0, 3, 17])
@pytest.mark.parametrize("combo", range(len(EDGE_COMBOS)))
@pytest.mark.parametrize("D,g", [(D, g) for D in (64, 128, 256) for g in (1, 2, 4, 8)])
def test_edges_balanced(D, g, combo, workers):
    bs, W, sinks, _ = EDGE_COMBOS[combo]
    wl = make_workload(name="edge", seq_lens=EDGE_LENS, num_q_heads=2 * g, num_kv_heads=2,
                       head_dim=D, block_size=bs, seed=[D, g, combo, 1], window=W,
                       with_sinks=sinks, poison=True)
    t = to_dev(wl)
    compare(*run_gpu(wl, t, partition_size=BALANCED, num_workers=workers), *oracle_full(wl),
            f"edge balanced workers={workers} D={D} g={g} bs={bs} W={W} sinks={sinks}")


def test_balanced_bad_tables_and_lengths():
    wl = make_workload(name="bad", seq_lens=[40, 40, 40, 33], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=[5])
    exp = oracle_full(wl)
    wl.block_table[1, 1] = wl.num_blocks
    wl.block_table[2, 0] = -7
    t = to_dev(wl)
    t["L"] = torch.tensor([40, 40, 40, 49], dtype=torch.int32, device="cuda")   # 49 > 3 * 16
    for workers in (0, 1, 5):
        out, lse = run_gpu(wl, t, partition_size=BALANCED, num_workers=workers)
        assert np.isnan(out[1:]).all() and np.isnan(lse[1:]).all(), workers
        assert np.abs(out[0] - exp[0][0]).max() < 1e-3


def test_balanced_repeat_bit_identical_and_lse_null():
    wl = make_config(5, seq_lens=[5000, 17, 9000, 4096, 4097, 1, 300, 0])
    t = to_dev(wl)
    a = run_gpu(wl, t, partition_size=BALANCED, num_workers=50)
    for _ in range(3):
        b = run_gpu(wl, t, partition_size=BALANCED, num_workers=50)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    out, lse = pa.decode_balanced(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                                  window=wl.window, sinks=t["sinks"], want_lse=False,
                                  num_workers=50)
    torch.cuda.synchronize()
    assert lse is None
    assert np.array_equal(out.cpu().numpy().astype(np.float64), a[0])


@pytest.mark.parametrize("hkv,g", [(1, 8), (2, 2), (4, 1)])
@pytest.mark.parametrize("workers", [997, 4096])
def test_balanced_many_pieces(hkv, g, workers):
    """Units cut into hundreds of pieces (long chains for the fix-up merge), next to short and
    empty sequences, with sinks."""
    wl = make_workload(name="long", seq_lens=[32768, 100, 0, 16384, 4097], num_q_heads=hkv * g,
                       num_kv_heads=hkv, head_dim=128, block_size=64, seed=[hkv, g, workers],
                       with_sinks=True, poison=True)
    t = to_dev(wl)
    a = run_gpu(wl, t, partition_size=BALANCED, num_workers=workers)
    compare(*a, *oracle_full(wl), f"many pieces Hkv={hkv} g={g} workers={workers}")
    b = run_gpu(wl, t, partition_size=BALANCED, num_workers=workers)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("schedule", ["balanced", "unsplit", "partitioned"])
def test_large_batch_of_short_sequences(schedule):
    """2048 sequences of 0..80 tokens (16384 (sequence, KV head) units, eight per worker and
    more), 32 q / 8 KV heads, window 50 and sinks: every unit in full against the oracle."""
    rng = np.random.default_rng(2048)
    lens = rng.integers(0, 81, size=2048)
    wl = make_workload(name="large batch", seq_lens=lens, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, block_size=16, seed=[2048], window=50, with_sinks=True,
                       poison=True)
    t = to_dev(wl)
    P = {"balanced": BALANCED, "unsplit": 0, "partitioned": 32}[schedule]
    out, lse = run_gpu(wl, t, partition_size=P)
    compare(out, lse, *oracle_full(wl), f"large batch B=2048 {schedule}")


@pytest.mark.parametrize("schedule", ["balanced", "partitioned"])
def test_widest_heads_largest_blocks(schedule):
    """head_dim 256, 64 q / 8 KV heads, 256-token blocks, one length around every block edge and
    one of 16384: every (sequence, head) row against the oracle."""
    wl = make_workload(name="widest", seq_lens=[16384, 1, 255, 256, 257, 9000, 0, 513],
                       num_q_heads=64, num_kv_heads=8, head_dim=256, block_size=256,
                       seed=[256, 64], window=0, with_sinks=True, poison=True)
    t = to_dev(wl)
    P = {"balanced": BALANCED, "partitioned": 512}[schedule]
    compare(*run_gpu(wl, t, partition_size=P), *oracle_full(wl),
            f"widest D=256 g=8 bs=256 {schedule}")

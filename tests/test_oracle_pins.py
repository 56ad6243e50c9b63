"""Pins for the fp64 oracle: each test checks it against something other than its own formula.

Closed forms, invariants, library routines (scipy's softmax/logsumexp on the unpaged layout), a
pure-Python brute force, and hand-derived values (tests/golden/hand_worked.json).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import brute, ref
from workloads import f32_to_bf16_bits, make_config, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def small(seq_lens, hq=4, hkv=2, d=16, bs=4, seed=11, **kw):
    return make_workload(name="pin", seq_lens=seq_lens, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, block_size=bs, seed=[seed], **kw)


def run(wl, **over):
    args = dict(window=wl.window, sinks=wl.sinks)
    args.update(over)
    return ref.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                      wl.block_size, **args)


def f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# (i) paged == dense softmax(q K^T scale) V on contiguous, unpaged tensors (scipy routines)
# ---------------------------------------------------------------------------------------------
def dense_via_scipy(q, K, V, scale, window=0, sinks=None, lens=None):
    """q [B][Hq][D] f64, K/V [B][Hkv][Lmax][D] f64 contiguous per sequence."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = lens[b]
        lo = max(0, L - window) if window else 0
        for h in range(Hq):
            kv = h * Hkv // Hq
            z = scale * (K[b, kv, lo:L] @ q[b, h])
            if sinks is not None:
                z = np.append(z, float(sinks[h]))
            if z.size == 0:
                continue
            p = softmax(z)
            out[b, h] = p[: L - lo] @ V[b, kv, lo:L]
            lse[b, h] = logsumexp(z)
    return out, lse


@pytest.mark.parametrize("window,with_sinks,hq,hkv", [(0, False, 4, 2), (5, False, 8, 2),
                                                    (0, True, 6, 3), (7, True, 4, 4),
                                                    (0, False, 8, 1)])
def test_paged_equals_dense_unpaged(window, with_sinks, hq, hkv):
    rng = np.random.default_rng(3)
    lens = [1, 4, 9, 23, 0, 17]
    B, D, bs = len(lens), 8, 4
    Lmax = max(lens)
    Kc = f32_to_bf16_bits(rng.standard_normal((B, hkv, Lmax, D)).astype(np.float32))
    Vc = f32_to_bf16_bits(rng.standard_normal((B, hkv, Lmax, D)).astype(np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((B, hq, D)).astype(np.float32))
    sinks = rng.standard_normal(hq).astype(np.float32) if with_sinks else None
    # scatter the contiguous rows into a shuffled page pool (the test's own paging)
    nblk = [-(-L // bs) for L in lens]
    pool = sum(nblk) + 3
    perm = rng.permutation(pool)
    k_cache = np.full((pool, hkv, bs, D), 0x7FC0, np.uint16)
    v_cache = np.full((pool, hkv, bs, D), 0x7FC0, np.uint16)
    bt = np.full((B, max(nblk)), perm[-1], np.int32)
    off = 0
    for b, L in enumerate(lens):
        for i in range(nblk[b]):
            phys = perm[off]
            off += 1
            bt[b, i] = phys
            n = min(bs, L - i * bs)
            k_cache[phys, :, :n] = Kc[b, :, i * bs:i * bs + n]
            v_cache[phys, :, :n] = Vc[b, :, i * bs:i * bs + n]
    scale = np.float32(0.37)
    out, lse = ref.decode(q, k_cache, v_cache, bt, np.array(lens, np.int32), scale, bs,
                          window=window, sinks=sinks)
    eo, el = dense_via_scipy(f64(q), f64(Kc), f64(Vc), float(scale), window,
                             None if sinks is None else sinks.astype(np.float64), lens)
    assert np.abs(out - eo).max() < 1e-12
    fin = np.isfinite(el)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - el[fin]).max() < 1e-12


# ---------------------------------------------------------------------------------------------
# (ii) invariance under any permutation of the physical blocks (table remapped)
# ---------------------------------------------------------------------------------------------
def test_block_permutation_invariance():
    wl = small([13, 40, 3, 29], window=0, with_sinks=True, poison=True)
    out, lse = run(wl)
    sigma = np.random.default_rng(5).permutation(wl.num_blocks)
    k2 = np.empty_like(wl.k_cache)
    v2 = np.empty_like(wl.v_cache)
    k2[sigma] = wl.k_cache
    v2[sigma] = wl.v_cache
    bt2 = sigma[wl.block_table].astype(np.int32)
    out2, lse2 = ref.decode(wl.q, k2, v2, bt2, wl.seq_lens, wl.scale, wl.block_size,
                            sinks=wl.sinks)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    assert np.isfinite(out).all()


# ---------------------------------------------------------------------------------------------
# special cases with closed forms
# ---------------------------------------------------------------------------------------------
def test_seq_len_one_returns_that_v_row_exactly():
    wl = small([1, 1, 1], poison=True)
    out, lse = run(wl)
    g = wl.group
    for b in range(3):
        phys = wl.block_table[b, 0]
        for h in range(wl.num_q_heads):
            vrow = f64(wl.v_cache[phys, h // g, 0])
            assert np.array_equal(out[b, h], vrow)
            l = float(wl.scale) * math.fsum(f64(wl.q[b, h]) * f64(wl.k_cache[phys, h // g, 0]))
            assert abs(lse[b, h] - l) < 1e-12


def test_identical_keys_give_mean_of_v():
    wl = small([1, 7, 33], poison=True)
    # every attended key of every sequence equals one fixed row
    key = wl.k_cache[wl.block_table[0, 0], 0, 0].copy()
    for b, L in enumerate(wl.seq_lens):
        for t in range(L):
            wl.k_cache[wl.block_table[b, t // wl.block_size], :, t % wl.block_size] = key
    out, lse = run(wl)
    for b, L in enumerate(wl.seq_lens):
        for h in range(wl.num_q_heads):
            kv = h // wl.group
            V = np.array([f64(wl.v_cache[wl.block_table[b, t // 4], kv, t % 4]) for t in range(L)])
            assert np.abs(out[b, h] - V.mean(axis=0)).max() < 1e-13
            l = float(wl.scale) * math.fsum(f64(wl.q[b, h]) * f64(key))
            assert abs(lse[b, h] - (l + math.log(L))) < 1e-12


def test_large_logits_identical_keys_give_mean_of_v():
    """Logits near 1000, far past where exp overflows in float64 (about 709): identical keys
    must still give the mean of V and lse = l + ln L.  Shift invariance of softmax is what
    makes this finite; evaluating exp(logit) without subtracting the max cannot."""
    wl = small([3, 16, 21], hq=2, hkv=1, d=16)
    key = f32_to_bf16_bits(f64(wl.q[0, 0]).astype(np.float32) * 256)   # exact: a power of two
    for b, L in enumerate(wl.seq_lens):
        for t in range(L):
            wl.k_cache[wl.block_table[b, t // wl.block_size], 0, t % wl.block_size] = key
    out, lse = run(wl)
    for b, L in enumerate(wl.seq_lens):
        V = np.array([f64(wl.v_cache[wl.block_table[b, t // 4], 0, t % 4]) for t in range(L)])
        l = float(wl.scale) * math.fsum(f64(wl.q[b, 0]) * f64(key))
        if b == 0:
            assert l > 800.0   # the case this pin is about
        assert np.abs(out[b, 0] - V.mean(axis=0)).max() < 1e-12
        assert abs(lse[b, 0] - (l + math.log(L))) < 1e-9


def test_scale_zero_gives_mean_over_window():
    wl = small([30, 12], window=9, poison=True)
    out, _ = run(wl)  # sanity: finite
    assert np.isfinite(out).all()
    out0, lse0 = ref.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, 0.0,
                            wl.block_size, window=9)
    for b, L in enumerate(wl.seq_lens):
        lo = max(0, L - 9)
        for h in range(wl.num_q_heads):
            V = np.array([f64(wl.v_cache[wl.block_table[b, t // 4], h // wl.group, t % 4])
                          for t in range(lo, L)])
            assert np.abs(out0[b, h] - V.mean(axis=0)).max() < 1e-13
            assert abs(lse0[b, h] - math.log(L - lo)) < 1e-13


def test_needle_key_selects_its_value():
    wl = small([50], hq=2, hkv=1, d=8)
    b, j = 0, 31
    phys, slot = wl.block_table[b, j // 4], j % 4
    wl.k_cache[phys, 0, slot] = f32_to_bf16_bits(f64(wl.q[b, 0]).astype(np.float32) * 64)
    out, _ = run(wl)
    assert np.abs(out[b, 0] - f64(wl.v_cache[phys, 0, slot])).max() < 1e-6


def test_v_all_ones():
    wl = small([5, 26], with_sinks=True)
    wl.v_cache[:] = 0x3F80
    out, lse = run(wl, sinks=None)
    assert np.abs(out - 1.0).max() < 1e-14
    out_s, lse_s = run(wl)
    expect = 1.0 - np.exp(wl.sinks.astype(np.float64)[None, :] - lse_s)
    assert np.abs(out_s - expect[..., None]).max() < 1e-14


def test_linearity_in_v():
    rng = np.random.default_rng(2)
    qv, K = rng.standard_normal(8), rng.standard_normal((19, 8))
    V1, V2 = rng.standard_normal((19, 8)), rng.standard_normal((19, 8))
    a, c = 0.75, -2.5
    o1, _ = ref.softmax_attention(qv, K, V1, 0.3, sink=0.2)
    o2, _ = ref.softmax_attention(qv, K, V2, 0.3, sink=0.2)
    o12, _ = ref.softmax_attention(qv, K, a * V1 + c * V2, 0.3, sink=0.2)
    assert np.abs(o12 - (a * o1 + c * o2)).max() < 1e-13


def test_empty_sequence():
    wl = small([0, 5], with_sinks=True)
    out, lse = run(wl, sinks=None)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.all(np.isneginf(lse[0]))
    out_s, lse_s = run(wl)
    assert np.array_equal(out_s[0], np.zeros_like(out_s[0]))
    assert np.allclose(lse_s[0], wl.sinks.astype(np.float64), atol=0, rtol=0)


# ---------------------------------------------------------------------------------------------
# window and sinks
# ---------------------------------------------------------------------------------------------
def test_window_ge_len_equals_no_window():
    wl = small([5, 16, 31], poison=True)
    a = run(wl, window=0)
    b = run(wl, window=31)
    c = run(wl, window=1000)
    for x, y in ((a, b), (a, c)):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])


def test_window_one_is_last_v_row():
    wl = small([5, 16, 31], window=1, poison=True)
    out, _ = run(wl)
    for b, L in enumerate(wl.seq_lens):
        t = L - 1
        for h in range(wl.num_q_heads):
            assert np.array_equal(out[b, h], f64(wl.v_cache[wl.block_table[b, t // 4],
                                                            h // wl.group, t % 4]))


def test_needle_just_outside_window_is_ignored():
    wl = small([40], hq=1, hkv=1, d=8, window=10)
    b = 0
    j_out, j_in = 40 - 11, 40 - 10
    base, _ = run(wl)
    big = f32_to_bf16_bits(f64(wl.q[b, 0]).astype(np.float32) * 64)
    wl.k_cache[wl.block_table[b, j_out // 4], 0, j_out % 4] = big
    same, _ = run(wl)
    assert np.array_equal(base, same)
    wl.k_cache[wl.block_table[b, j_in // 4], 0, j_in % 4] = big
    hit, _ = run(wl)
    assert np.abs(hit[b, 0] - f64(wl.v_cache[wl.block_table[b, j_in // 4], 0, j_in % 4])).max() < 1e-6


def test_sink_minus_huge_equals_no_sink():
    wl = small([9, 22], with_sinks=True)
    out, lse = run(wl, sinks=None)
    out2, lse2 = run(wl, sinks=np.full(wl.num_q_heads, -1e30, np.float32))
    assert np.abs(out - out2).max() < 1e-15 and np.abs(lse - lse2).max() < 1e-15


def test_sink_single_token_logistic():
    wl = small([1, 1], with_sinks=True)
    out, lse = run(wl)
    for b in range(2):
        phys = wl.block_table[b, 0]
        for h in range(wl.num_q_heads):
            kv = h // wl.group
            l = float(wl.scale) * math.fsum(f64(wl.q[b, h]) * f64(wl.k_cache[phys, kv, 0]))
            s = float(wl.sinks[h])
            sig = 1.0 / (1.0 + math.exp(s - l))
            assert np.abs(out[b, h] - sig * f64(wl.v_cache[phys, kv, 0])).max() < 1e-13
            assert abs(lse[b, h] - np.logaddexp(l, s)) < 1e-13


# ---------------------------------------------------------------------------------------------
# GQA == MHA with the KV heads repeated
# ---------------------------------------------------------------------------------------------
def test_gqa_equals_mha_with_repeated_kv_heads():
    wl = small([11, 35], hq=8, hkv=2, window=13, with_sinks=True)
    out, lse = run(wl)
    rep_k = np.repeat(wl.k_cache, wl.group, axis=1)
    rep_v = np.repeat(wl.v_cache, wl.group, axis=1)
    out2, lse2 = ref.decode(wl.q, rep_k, rep_v, wl.block_table, wl.seq_lens, wl.scale,
                            wl.block_size, window=13, sinks=wl.sinks)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------------------------------------
# split-KV + LSE merge == unsplit
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("P,window,with_sinks", [(4, 0, False), (8, 0, True), (8, 13, True),
                                                 (12, 6, True), (64, 0, True), (4, 1, False)])
def test_split_merge_equals_unsplit(P, window, with_sinks):
    wl = small([0, 1, 3, 4, 5, 17, 40, 63], window=window, with_sinks=with_sinks, poison=True)
    out, lse = run(wl)
    o, l = ref.decode_partitions(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                 wl.scale, wl.block_size, P, window=window, sinks=wl.sinks)
    counts = np.array([ref.num_partitions(int(L), P) for L in wl.seq_lens])
    m_out, m_lse = ref.merge_partitions(o, l, counts)
    assert np.abs(m_out - out).max() < 1e-12
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(m_lse), fin)
    assert np.abs(m_lse[fin] - lse[fin]).max() < 1e-12
    # one partition covering everything is the identity
    o1, l1 = ref.decode_partitions(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                   wl.scale, wl.block_size, 1 << 20, window=window,
                                   sinks=wl.sinks)
    assert np.array_equal(o1[:, :, 0], out) and np.array_equal(l1[:, :, 0], lse)


def test_merge_skips_empty_slots():
    o = np.zeros((1, 1, 3, 2))
    o[0, 0, 0] = [np.nan, np.nan]     # an empty slot's o is never read
    o[0, 0, 1] = [1.0, 2.0]
    o[0, 0, 2] = [3.0, 4.0]
    l = np.array([[[-np.inf, math.log(1.0), math.log(3.0)]]])
    out, lse = ref.merge_partitions(o, l, np.array([3]))
    assert np.abs(out[0, 0] - np.array([2.5, 3.5])).max() < 1e-15
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


# ---------------------------------------------------------------------------------------------
# brute force on tiny inputs (pure Python, no max subtraction, struct-decoded bf16)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("window", [0, 1, 3, 8])
@pytest.mark.parametrize("with_sinks", [False, True])
@pytest.mark.parametrize("hq,hkv,d,bs", [(2, 1, 4, 2), (3, 3, 8, 4), (4, 2, 2, 8)])
def test_brute_force_tiny(window, with_sinks, hq, hkv, d, bs):
    wl = make_workload(name="tiny", seq_lens=[1, 2, 7, 16, 33, 0], num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=[hq, d, bs, window],
                       window=window, with_sinks=with_sinks, poison=True)
    out, lse = run(wl)
    qL, kL, vL = wl.q.tolist(), wl.k_cache.tolist(), wl.v_cache.tolist()
    btL = wl.block_table.tolist()
    sinks = None if wl.sinks is None else wl.sinks.tolist()
    for b in range(wl.num_seqs):
        for h in range(hq):
            bo, bl = brute.decode_head(qL, kL, vL, btL, wl.seq_lens.tolist(), float(wl.scale),
                                       bs, b, h, window=window, sinks=sinks)
            assert np.abs(out[b, h] - np.array(bo)).max() < 1e-12
            if math.isinf(bl):
                assert math.isinf(lse[b, h]) and lse[b, h] < 0
            else:
                assert abs(lse[b, h] - bl) < 1e-12


# ---------------------------------------------------------------------------------------------
# hand-derived worked example
# ---------------------------------------------------------------------------------------------
def load_golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    i = g["inputs"]
    q = np.array(i["q_bits"], np.uint16)
    k = np.array(i["k_blocks_bits"], np.uint16)
    v = np.array(i["v_blocks_bits"], np.uint16)
    bt = np.array(i["block_table"], np.int32)
    L = np.array(i["seq_lens"], np.int32)
    return g, q, k, v, bt, L, np.float32(i["scale"]), i["block_size"]


def test_hand_worked_golden():
    g, q, k, v, bt, L, scale, bs = load_golden()
    tol = g["tolerance"]
    for case in g["cases"]:
        sinks = None if case["sinks"] is None else np.array(case["sinks"], np.float32)
        out, lse = ref.decode(q, k, v, bt, L, scale, bs, window=case["window"], sinks=sinks)
        assert np.abs(out - np.array(case["out"])).max() < tol, case["name"]
        assert np.abs(lse - np.array(case["lse"])).max() < tol, case["name"]
    sp = g["split"]
    o, l = ref.decode_partitions(q, k, v, bt, L, scale, bs, sp["partition_size"])
    assert np.abs(o[0, sp["head"]] - np.array(sp["o"])).max() < tol
    assert np.abs(l[0, sp["head"]] - np.array(sp["lse"])).max() < tol


# ---------------------------------------------------------------------------------------------
# the seeded workloads themselves (integer structure, bit-exact)
# ---------------------------------------------------------------------------------------------
def test_config1_structure():
    wl = make_config(1, poison=True)
    assert wl.num_blocks == 32 and list(wl.seq_lens) == [37, 100]
    assert wl.block_table.shape == (2, 7)
    used = list(wl.block_table[0, :3]) + list(wl.block_table[1, :7])
    assert len(set(used)) == 10 and all(0 <= x < 32 for x in used)
    out, lse = run(wl)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_config2_lengths_and_pool():
    L = make_config.__globals__["config_seq_lens"](2)
    assert L.shape == (64,) and L.min() >= 512 and L.max() <= 4096
    need = int(sum(-(-int(x) // 16) for x in L))
    from workloads import pool_blocks
    assert pool_blocks(L, 16) == math.ceil(1.1 * need)


def test_config5_lengths():
    from workloads import config_seq_lens
    L = config_seq_lens(5)
    assert L.shape == (128,) and L.min() >= 1 and L.max() <= 32768
    assert 1200 < np.median(L) < 3500


# ---------------------------------------------------------------------------------------------
# FP8 E4M3 KV cache
# ---------------------------------------------------------------------------------------------
def test_fp8_e4m3_decoding_matches_torch():
    """All 256 codes against torch's float8_e4m3fn (a library decoding of the OCP format)."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    mine = ref.fp8_e4m3_bits_to_f64(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])
    assert np.isnan(mine).sum() == 2 and mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def _fp8_workload(scales, **kw):
    d = dict(name="fp8", seq_lens=[37, 100, 1, 0], num_q_heads=8, num_kv_heads=2, head_dim=64,
             block_size=16, seed=[41], kv_format="fp8_e4m3", kv_scales=scales)
    d.update(kw)
    return make_workload(**d)


def _decode(wl, scale=None, **over):
    kw = dict(window=wl.window, sinks=wl.sinks, kv_format=wl.kv_format, k_scale=wl.k_scale,
              v_scale=wl.v_scale)
    kw.update(over)
    return ref.decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                      wl.scale if scale is None else scale, wl.block_size, **kw)


def test_fp8_attention_equals_bf16_attention_on_dequantized_values():
    """With power-of-two scales every dequantised value is exact in bf16, so the FP8 path must
    equal the bf16 definition applied to those values."""
    wl = _fp8_workload((0.0625, 0.125), window=64, with_sinks=True)
    o8, l8 = _decode(wl)
    kb = f32_to_bf16_bits((ref.fp8_e4m3_bits_to_f64(wl.k_cache) * 0.0625).astype(np.float32))
    vb = f32_to_bf16_bits((ref.fp8_e4m3_bits_to_f64(wl.v_cache) * 0.125).astype(np.float32))
    assert np.array_equal(ref.bf16_bits_to_f64(kb), ref.fp8_e4m3_bits_to_f64(wl.k_cache) * 0.0625)
    ob, lb = ref.decode(wl.q, kb, vb, wl.block_table, wl.seq_lens, wl.scale, wl.block_size,
                        window=wl.window, sinks=wl.sinks)
    np.testing.assert_allclose(o8, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, lb, rtol=0, atol=1e-12)


def test_fp8_scales_act_as_closed_forms():
    """v_scale multiplies the output and leaves the LSE alone; k_scale multiplies every logit,
    which is the same as multiplying the attention scale."""
    wl = _fp8_workload((1.0, 1.0))
    o1, l1 = _decode(wl)
    o2, l2 = _decode(wl, v_scale=0.5)
    assert np.abs(o2 - 0.5 * o1).max() <= 1e-12
    assert np.array_equal(l1, l2)
    o3, l3 = _decode(wl, k_scale=0.25)
    o4, l4 = _decode(wl, scale=np.float32(wl.scale) * np.float32(0.25))
    np.testing.assert_allclose(o3, o4, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=0, atol=1e-12)   # -inf for the empty sequence


# ---------------------------------------------------------------------------------------------
# several query tokens per sequence (decode_multi): causal, each token at position L - Q + i
# ---------------------------------------------------------------------------------------------
def run_multi(wl, **over):
    args = dict(window=wl.window, sinks=wl.sinks)
    args.update(over)
    return ref.decode_multi(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
                            wl.block_size, **args)


def test_multi_with_one_token_is_decode():
    wl = small([1, 4, 9, 23, 0, 17], window=5, with_sinks=True)
    o1, l1 = run(wl)
    om, lm = ref.decode_multi(wl.q[:, None], wl.k_cache, wl.v_cache, wl.block_table,
                              wl.seq_lens, wl.scale, wl.block_size, window=wl.window,
                              sinks=wl.sinks)
    assert np.array_equal(om[:, 0], o1) and np.array_equal(lm[:, 0], l1)


@pytest.mark.parametrize("Q,window,with_sinks", [(2, 0, False), (3, 0, True), (4, 5, False),
                                                 (5, 3, True), (8, 1, False)])
def test_multi_equals_dense_causal_masked_softmax(Q, window, with_sinks):
    """Against the textbook masked form on unpaged tensors: S = scale Q K^T [Q x L], masked
    where key t lies after the query's position or before its window, softmax by rows (scipy),
    times V."""
    lens = [Q + 6, 1, 23, Q, 17]
    wl = small(lens, hq=4, hkv=2, d=8, bs=4, seed=29, q_len=Q, window=window,
               with_sinks=with_sinks)
    out, lse = run_multi(wl)
    for b, L in enumerate(lens):
        for kvh in range(2):
            Kd = f64(ref.gather_rows(wl.k_cache, wl.block_table, b, kvh, 0, L, wl.block_size))
            Vd = f64(ref.gather_rows(wl.v_cache, wl.block_table, b, kvh, 0, L, wl.block_size))
            t = np.arange(L)
            pos = L - Q + np.arange(Q)
            allowed = t[None, :] <= pos[:, None]
            if window > 0:
                allowed &= t[None, :] > pos[:, None] - window
            for h in range(2 * kvh, 2 * kvh + 2):
                S = float(wl.scale) * (f64(wl.q[b, :, h]) @ Kd.T)
                S = np.where(allowed, S, -np.inf)
                if with_sinks:
                    S = np.concatenate([S, np.full((Q, 1), float(wl.sinks[h]))], axis=1)
                for i in range(Q):
                    if not np.isfinite(S[i]).any():
                        assert lse[b, i, h] == -np.inf and not out[b, i, h].any()
                        continue
                    p = softmax(S[i])
                    assert np.abs(out[b, i, h] - p[:L] @ Vd).max() < 1e-12
                    assert abs(lse[b, i, h] - logsumexp(S[i])) < 1e-12


def test_multi_token_equals_decode_of_its_prefix():
    """Query token i of Q sees exactly what a one-token decode of the first L - Q + i + 1
    tokens sees (the causal rule)."""
    Q = 4
    lens = [9, 23, 4, 2]
    wl = small(lens, hq=4, hkv=2, d=8, bs=4, seed=31, q_len=Q, window=6, with_sinks=True)
    out, lse = run_multi(wl)
    for i in range(Q):
        prefix = np.maximum(wl.seq_lens - Q + i + 1, 0).astype(np.int32)
        o1, l1 = ref.decode(wl.q[:, i], wl.k_cache, wl.v_cache, wl.block_table, prefix,
                            wl.scale, wl.block_size, window=wl.window, sinks=wl.sinks)
        assert np.array_equal(out[:, i], o1) and np.array_equal(lse[:, i], l1), i


def test_multi_positions_before_the_sequence_attend_nothing():
    Q = 4
    wl = small([2, 0], hq=2, hkv=1, d=4, bs=4, seed=5, q_len=Q, with_sinks=True)
    out, lse = run_multi(wl)
    # sequence 0: tokens 0 and 1 sit at positions -2 and -1, tokens 2 and 3 at 0 and 1
    for b, first_real in ((0, 2), (1, Q)):
        for i in range(first_real):
            assert not out[b, i].any()
            assert np.array_equal(lse[b, i], wl.sinks.astype(np.float64))
    assert np.isfinite(lse[0, 2:]).all() and out[0, 2:].any()


@pytest.mark.parametrize("Q,window,with_sinks", [(2, 0, True), (3, 2, False), (4, 3, True)])
def test_multi_brute_force_tiny(Q, window, with_sinks):
    wl = small([Q + 5, 3, Q], hq=2, hkv=1, d=4, bs=2, seed=37, q_len=Q, window=window,
               with_sinks=with_sinks)
    out, lse = run_multi(wl)
    q = wl.q.tolist()
    k = wl.k_cache.tolist()
    v = wl.v_cache.tolist()
    bt = wl.block_table.tolist()
    for b in range(wl.num_seqs):
        for i in range(Q):
            for h in range(wl.num_q_heads):
                eo, el = brute.decode_head_multi(q, k, v, bt, wl.seq_lens.tolist(),
                                                 float(wl.scale), wl.block_size, b, i, h, Q,
                                                 window, None if wl.sinks is None
                                                 else wl.sinks.tolist())
                assert np.abs(out[b, i, h] - np.array(eo)).max() < 1e-12
                assert (lse[b, i, h] == el == -math.inf) or abs(lse[b, i, h] - el) < 1e-12


def test_multi_workload_poison_spares_every_query_window():
    """The generator's poison must leave every key some query token attends finite."""
    Q, W = 3, 5
    wl = small([20, 9, 3], hq=2, hkv=1, d=4, bs=4, seed=41, q_len=Q, window=W, poison=True)
    out, lse = run_multi(wl)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert wl.attended_tokens().tolist() == [min(20, W + Q - 1), min(9, W + Q - 1), 3]

"""Pins for the oracle's row-by-row entry points (CPU only).

ref.decode_one, and the sampled-row helpers built on it, check the GPU path wherever a workload
is too large to run the whole-batch oracle at every test.  Each is pinned here against the
whole-batch functions (ref.decode, ref.decode_multi), which are themselves pinned against the
dense definition, a brute force and closed forms (test_oracle_pins.py): every (sequence, head)
row must come out bit for bit the same, over group sizes 1/4/8, windows, sinks, FP8 scales and
the lengths around a block boundary, so that a slip confined to the row entry point (a sink read
by KV head, a window edge, a wrong KV head) fails here.
"""
import numpy as np
import pytest

from oracle import ref
from tests.oracle_rows import oracle_multi_triples, oracle_pairs
from workloads import make_workload

BS = 4
# around the block boundary: empty, one token, a full block, one past it, and longer
LENS = [0, 1, BS, BS + 1, 2 * BS - 1, 23, 37]


def _wl(hq, hkv, window, sinks, kv="bf16", q_len=1, seed=3):
    scales = (0.375, -1.25) if kv == "fp8_e4m3" else (1.0, 1.0)
    return make_workload(name="rows", seq_lens=LENS, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=8, block_size=BS, seed=[seed, hq, hkv, window],
                         window=window, with_sinks=sinks, kv_format=kv, kv_scales=scales,
                         q_len=q_len, poison=True)


def _whole(wl):
    kw = dict(window=wl.window, sinks=wl.sinks, kv_format=wl.kv_format, k_scale=wl.k_scale,
              v_scale=wl.v_scale)
    fn = ref.decode_multi if wl.q_len > 1 else ref.decode
    return fn(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.scale,
              wl.block_size, **kw)


def _same(a, b):
    return np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("window", [0, 1, 5])
@pytest.mark.parametrize("sinks", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (16, 2)])
def test_decode_one_equals_decode_row_by_row(hq, hkv, window, sinks, kv):
    wl = _wl(hq, hkv, window, sinks, kv)
    out, lse = _whole(wl)
    for b in range(wl.num_seqs):
        for h in range(hq):
            o, l = ref.decode_one(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                                  wl.scale, wl.block_size, b, h, window=wl.window,
                                  sinks=wl.sinks, kv_format=wl.kv_format, k_scale=wl.k_scale,
                                  v_scale=wl.v_scale)
            assert _same(o, out[b, h]) and _same(l, lse[b, h]), (b, h)


def test_oracle_pairs_equals_decode():
    wl = _wl(8, 2, 5, True)
    out, lse = _whole(wl)
    pairs = [(b, h) for b in range(wl.num_seqs) for h in range(wl.num_q_heads)]
    po, pl = oracle_pairs(wl, pairs)
    for i, (b, h) in enumerate(pairs):
        assert _same(po[i], out[b, h]) and _same(pl[i], lse[b, h]), (b, h)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("q_len,window,sinks", [(2, 0, False), (3, 5, True), (5, 1, True),
                                                (8, 0, True)])
def test_multi_triples_equal_decode_multi(q_len, window, sinks, kv):
    wl = _wl(8, 2, window, sinks, kv, q_len=q_len, seed=9)
    out, lse = _whole(wl)
    triples = [(b, i, h) for b in range(wl.num_seqs) for i in range(q_len)
               for h in range(wl.num_q_heads)]
    to, tl = oracle_multi_triples(wl, triples)
    for n, (b, i, h) in enumerate(triples):
        assert _same(to[n], out[b, i, h]) and _same(tl[n], lse[b, i, h]), (b, i, h)

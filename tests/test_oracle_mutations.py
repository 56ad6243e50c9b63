"""Mutation checks: a plausible mistake planted in the oracle (on the CPU) must fail a pin.

Each case patches one oracle step, runs the pins that should catch it, and requires at least one
of them to fail; the oracle is restored afterwards by monkeypatch.
"""
import math

import numpy as np
import pytest

import tests.test_oracle_pins as pins
import tests.test_oracle_rows as rows
from oracle import ref


def _fails(fn, *args):
    try:
        fn(*args)
    except Exception:   # a failed assertion or a crash: either way the pin rejects it
        return True
    return False


def _wrong_kv_head(h, num_q_heads, num_kv_heads):
    # interleaved instead of consecutive grouping
    return h % num_kv_heads


def _window_off_by_one(L, window):
    start = max(0, L - window + 1) if window > 0 else 0
    return start, L


def _slot_off_by_one(cache, block_table, b, kvh, start, stop, block_size):
    t = np.arange(start, max(start, stop), dtype=np.int64)
    phys = block_table[b, t // block_size].astype(np.int64)
    return np.ascontiguousarray(cache[phys, kvh, (t + 1) % block_size, :])


_orig_softmax = ref.softmax_attention


def _sink_dropped(qv, K, V, scale, sink=None):
    return _orig_softmax(qv, K, V, scale, None)


def _scale_ignored(qv, K, V, scale, sink=None):
    return _orig_softmax(qv, K, V, 1.0, sink)


_orig_merge = ref.merge_partitions


def _merge_drops_last(o, lse, counts):
    return _orig_merge(o, lse, np.maximum(np.asarray(counts) - 1, 1))


def _causal_off_by_one(L, q_len, i, window):
    # the query's own key left out
    p = L - q_len + i
    if p < 0:
        return 0, 0
    start = max(0, p + 1 - window) if window > 0 else 0
    return start, p


def _max_not_subtracted(qv, K, V, scale, sink=None):
    # exp of the raw logits: the same function until a logit passes float64's exp range
    D = V.shape[1] if V.ndim == 2 else qv.shape[0]
    logits = scale * (K @ qv) if K.shape[0] else np.zeros(0)
    if not logits.size and sink is None:
        return np.zeros(D), -math.inf
    w = np.exp(logits)
    Z = float(w.sum()) + (math.exp(float(sink)) if sink is not None else 0.0)
    out = (w @ V) / Z if K.shape[0] else np.zeros(D)
    return out, math.log(Z)


def _block_and_slot_transposed(cache, block_table, b, kvh, start, stop, block_size):
    # the table indexed by the slot and the block read at the logical block index
    t = np.arange(start, max(start, stop), dtype=np.int64)
    phys = block_table[b, (t % block_size) % block_table.shape[1]].astype(np.int64)
    return np.ascontiguousarray(cache[phys, kvh, (t // block_size) % block_size, :])


def _tail_dropped(cache, block_table, b, kvh, start, stop, block_size):
    # only whole blocks: the partly filled last block of the sequence is left out
    stop = max(start, stop - stop % block_size)
    t = np.arange(start, stop, dtype=np.int64)
    phys = block_table[b, t // block_size].astype(np.int64)
    return np.ascontiguousarray(cache[phys, kvh, t % block_size, :])


_orig_decode_one = ref.decode_one


def _decode_one_sink_by_kv_head(q, k_cache, v_cache, block_table, seq_lens, scale, block_size,
                                b, h, window=0, sinks=None, **kw):
    if sinks is not None:
        g = q.shape[1] // k_cache.shape[1]
        sinks = np.repeat(np.asarray(sinks)[::g], g)   # the first head of each group's sink
    return _orig_decode_one(q, k_cache, v_cache, block_table, seq_lens, scale, block_size, b, h,
                            window=window, sinks=sinks, **kw)


def _decode_one_window_ignored(q, k_cache, v_cache, block_table, seq_lens, scale, block_size,
                               b, h, window=0, **kw):
    return _orig_decode_one(q, k_cache, v_cache, block_table, seq_lens, scale, block_size, b, h,
                            window=0, **kw)


MUTATIONS = {
    "gqa head map interleaved": ("kv_head_of", _wrong_kv_head,
                           [(pins.test_paged_equals_dense_unpaged, 0, False, 8, 2),
                            (pins.test_gqa_equals_mha_with_repeated_kv_heads,)]),
    "window off by one": ("attended_range", _window_off_by_one,
                          [(pins.test_window_one_is_last_v_row,),
                           (pins.test_paged_equals_dense_unpaged, 5, False, 8, 2)]),
    "slot index off by one": ("gather_rows", _slot_off_by_one,
                              [(pins.test_paged_equals_dense_unpaged, 0, False, 4, 2),
                               (pins.test_hand_worked_golden,)]),
    "sink dropped": ("softmax_attention", _sink_dropped,
                     [(pins.test_sink_single_token_logistic,),
                      (pins.test_hand_worked_golden,)]),
    "max not subtracted": ("softmax_attention", _max_not_subtracted,
                           [(pins.test_large_logits_identical_keys_give_mean_of_v,)]),
    "block and slot index transposed": ("gather_rows", _block_and_slot_transposed,
                                        [(pins.test_paged_equals_dense_unpaged, 0, False, 4, 2),
                                         (pins.test_hand_worked_golden,)]),
    "tail of the last block dropped": ("gather_rows", _tail_dropped,
                                       [(pins.test_paged_equals_dense_unpaged, 0, False, 4, 2),
                                        (pins.test_seq_len_one_returns_that_v_row_exactly,)]),
    "decode_one sink read by KV head": ("decode_one", _decode_one_sink_by_kv_head,
                                        [(rows.test_decode_one_equals_decode_row_by_row, 8, 2, 0,
                                          True, "bf16"),
                                         (rows.test_oracle_pairs_equals_decode,)]),
    "decode_one window ignored": ("decode_one", _decode_one_window_ignored,
                                  [(rows.test_decode_one_equals_decode_row_by_row, 4, 4, 5,
                                    False, "bf16"),
                                   (rows.test_multi_triples_equal_decode_multi, 3, 5, True,
                                    "bf16")]),
    "scale ignored": ("softmax_attention", _scale_ignored,
                      [(pins.test_paged_equals_dense_unpaged, 0, False, 4, 2),
                       (pins.test_hand_worked_golden,)]),
    "merge drops last partition": ("merge_partitions", _merge_drops_last,
                                   [(pins.test_split_merge_equals_unsplit, 8, 0, True)]),
    "multi-token causal bound off by one": ("query_range", _causal_off_by_one,
                                            [(pins.test_multi_equals_dense_causal_masked_softmax,
                                              3, 0, True),
                                             (pins.test_multi_brute_force_tiny, 2, 0, True)]),
}


_orig_rows = ref.kv_rows_to_f64


def _fp8_bias_off_by_one(bits):
    c = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 8))
    return np.where((c >> 7) == 1, -1.0, 1.0) * np.where((e == 15) & (m == 7), np.nan, mag)


def _fp8_scale_ignored(rows, kv_format, scale):
    return _orig_rows(rows, kv_format, 1.0)


MUTATIONS.update({
    "fp8 exponent bias off by one": ("fp8_e4m3_bits_to_f64", _fp8_bias_off_by_one,
                                     [(pins.test_fp8_e4m3_decoding_matches_torch,)]),
    "fp8 scale ignored": ("kv_rows_to_f64", _fp8_scale_ignored,
                          [(pins.test_fp8_scales_act_as_closed_forms,),
                           (pins.test_fp8_attention_equals_bf16_attention_on_dequantized_values,)]),
})


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad, checks = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, bad)
    caught = [_fails(c[0], *c[1:]) for c in checks]
    assert all(caught), f"mutation '{name}' escaped: {caught}"


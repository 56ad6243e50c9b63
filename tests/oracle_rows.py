"""Row-by-row oracle results for the GPU parity tests: one (sequence, head) or one (sequence,
query token, head) at a time, so that a large workload can be checked at sampled rows.  Only
NumPy and the oracle are imported, so the CPU tests can pin these against the whole-batch
oracle functions (tests/test_oracle_rows.py)."""
from __future__ import annotations

import numpy as np

from oracle import ref


def oracle_pairs(wl, pairs):
    """Oracle (out, lse) of the (sequence b, query head h) pairs, each by ref.decode_one."""
    outs, lses = [], []
    for b, h in pairs:
        o, l = ref.decode_one(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                              wl.scale, wl.block_size, b, h, window=wl.window, sinks=wl.sinks,
                              kv_format=wl.kv_format, k_scale=wl.k_scale, v_scale=wl.v_scale)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)


def oracle_multi_triples(wl, triples):
    """Oracle rows of (sequence, query token, head) triples, one by one (q_len > 1): each is the
    one-token decode of the sequence's first L - q_len + i + 1 tokens (the causal rule)."""
    outs, lses = [], []
    Q = wl.q_len
    for b, i, h in triples:
        L = int(wl.seq_lens[b])
        prefix = np.array([max(L - Q + i + 1, 0)], np.int32)
        o, l = ref.decode_one(wl.q[b:b + 1, i], wl.k_cache, wl.v_cache, wl.block_table[b:b + 1],
                              prefix, wl.scale, wl.block_size, 0, h, window=wl.window,
                              sinks=wl.sinks, kv_format=wl.kv_format, k_scale=wl.k_scale,
                              v_scale=wl.v_scale)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)

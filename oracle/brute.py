"""Pure-Python brute-force paged-attention decode for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/ref.py for who may use it).  It pins the NumPy oracle by an
independent route: Python floats and math.exp, no NumPy, no max subtraction (inputs are tiny, so
exp(logit) cannot overflow), bf16 decoded with struct, every gather done token by token.

It computes the same quantity as oracle/ref.py: the softmax-weighted mean of the attended value
rows with an optional sink logit (randomvariable/vllm issue #23, "Attention parity", table
"Current state"), and the natural log of the softmax denominator used by split-KV reducers
(ROCm/rocm-libraries PR #13700, "prepare saved paged decode bindings once", Summary).
"""
from __future__ import annotations

import math
import struct


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def f32(x: float) -> float:
    """Round a Python float to the nearest fp32 (the scale and sinks are fp32 arguments)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def decode_head(q, k_cache, v_cache, block_table, seq_lens, scale, block_size, b, h,
                window=0, sinks=None):
    """(out row as a list, lse) for query head h of sequence b.

    Arguments are nested Python lists (or anything indexable) of bf16 bits:
    q[b][h][d], k_cache[blk][kvh][slot][d], v_cache likewise; block_table[b][i]; seq_lens[b]."""
    Hq = len(q[b])
    Hkv = len(k_cache[0])
    group = Hq // Hkv
    kvh = h // group
    D = len(q[b][h])
    L = int(seq_lens[b])
    first = L - window if (window > 0 and L > window) else 0
    sc = f32(scale)
    weights = []
    rows = []
    for t in range(first, L):
        blk = int(block_table[b][t // block_size])
        slot = t % block_size
        dot = 0.0
        for d in range(D):
            dot += bf16_to_float(q[b][h][d]) * bf16_to_float(k_cache[blk][kvh][slot][d])
        weights.append(math.exp(sc * dot))
        rows.append([bf16_to_float(v_cache[blk][kvh][slot][d]) for d in range(D)])
    Z = sum(weights)
    if sinks is not None:
        Z += math.exp(f32(sinks[h]))
    if Z == 0.0:
        return [0.0] * D, -math.inf
    out = [0.0] * D
    for w, row in zip(weights, rows):
        for d in range(D):
            out[d] += w * row[d]
    return [x / Z for x in out], math.log(Z)


def decode_head_multi(q, k_cache, v_cache, block_table, seq_lens, scale, block_size, b, i, h,
                      q_len, window=0, sinks=None):
    """(out row, lse) for query token i (of q_len) and head h of sequence b, q[b][i][h][d].

    The token sits at position L - q_len + i of the L tokens (new ones included) and sees the
    keys at or before it, the last `window` of them when window > 0."""
    Hq = len(q[b][i])
    Hkv = len(k_cache[0])
    kvh = h // (Hq // Hkv)
    D = len(q[b][i][h])
    pos = int(seq_lens[b]) - q_len + i
    sc = f32(scale)
    weights, rows = [], []
    for t in range(0, pos + 1):
        if window > 0 and t <= pos - window:
            continue
        blk = int(block_table[b][t // block_size])
        slot = t % block_size
        dot = 0.0
        for d in range(D):
            dot += bf16_to_float(q[b][i][h][d]) * bf16_to_float(k_cache[blk][kvh][slot][d])
        weights.append(math.exp(sc * dot))
        rows.append([bf16_to_float(v_cache[blk][kvh][slot][d]) for d in range(D)])
    Z = sum(weights)
    if sinks is not None:
        Z += math.exp(f32(sinks[h]))
    if Z == 0.0:
        return [0.0] * D, -math.inf
    out = [0.0] * D
    for w, row in zip(weights, rows):
        for d in range(D):
            out[d] += w * row[d]
    return [x / Z for x in out], math.log(Z)

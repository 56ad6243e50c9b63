"""fp64 CPU oracle for single-token paged-attention decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg may
import this module; the product path (the HIP library and its Python binding) never does.  It
shares no code, table or helper with the HIP path: it is plain NumPy in float64, written from the
definition of the operation, with no blocking or fusion beyond what the definition states.

What it computes, and where the pages define it:

* One-token decode over a paged KV cache, with split-KV partitions that each emit a partial
  output and a log-sum-exp merged by a reducer: ROCm/rocm-libraries PR #13700, "prepare saved
  paged decode bindings once", Summary and the review finding N1 (the reducer consumes the output,
  the sequence lengths and, when emitted, the LSE buffer).
* Online (running max/sum) softmax reaches the same function as a plain softmax, only in a
  different reduction order: vllm.cpp PR #564, "spec(BACKEND-ROCM): the ROCm head_dim=128 decode
  arm", section "It is a mirror of merged work, not new design".  So the oracle is the plain
  softmax definition.
* Grouped-query sharing (qg query heads per KV head): vllm.cpp PR #564, "What is deliberately not
  here" (qg=2/4/8 GQA fusion).
* Sliding window with out-of-window blocks skipped, and attention sinks as attention types:
  randomvariable/vllm issue #23, "Attention parity", table "Current state".

Readings where the pages are silent (each is listed with its reason in the design notes):
  KV layout [num_blocks][Hkv][block_size][D]; token t of sequence b lives at
  (block_table[b][t // block_size], t % block_size); q head h reads KV head h // (Hq/Hkv);
  the window keeps the last min(L, W) tokens, t in [L-W, L); a sink is one extra logit per q head
  that joins the max and the denominator with a zero value row; lse is the natural log of the full
  denominator (sink included); split partitions are absolute-aligned [pP, (p+1)P) intersected with
  the attended range, a sequence has max(1, ceil(L/P)) of them, the sink is folded into the first
  non-empty one (floor(start/P)), and an empty partition has lse = -inf and o = 0;
  L = 0 gives out = 0 and lse = -inf (lse = sink with a sink).

An FP8 KV cache (the 8-bit sibling of the bf16 path, named but not specified by the PR #13700
page above) is read as OCP FP8 E4M3 codes with one fp32 scale for K and one for V: the real
value of a stored code is its E4M3 value times the scale.  Everything after dequantisation is
the same definition.

Several new query tokens per sequence (decode_multi): the PR #13700 page's benchmark takes a
query length (its decode runs use one), and vllm.cpp PR #564, "What is deliberately not here",
leaves the longer-query case (prefill) out.  Reading: with q_len = Q new tokens and a sequence
length L that counts them, query token i sits at position p = L - Q + i and attends causally,
keys t <= p, within its own window [p + 1 - W, p] when W > 0; a position p < 0 attends nothing.
One token (Q = 1) is the decode above.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

NEG_INF = -math.inf


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: bf16 is the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def fp8_e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, exactly.  A code is sign | 4-bit exponent (bias 7)
    | 3-bit mantissa: exponent 0 is subnormal, m/8 * 2^-6; S.1111.111 is NaN; there are no
    infinities (the largest finite magnitude is 1.75 * 2^8 = 448)."""
    c = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def kv_rows_to_f64(rows: np.ndarray, kv_format: str, scale: float) -> np.ndarray:
    """Gathered cache rows -> float64 values: bf16 bit patterns as they are, FP8 E4M3 codes
    times the tensor's fp32 scale."""
    if kv_format == "bf16":
        return bf16_bits_to_f64(rows)
    if kv_format == "fp8_e4m3":
        return fp8_e4m3_bits_to_f64(rows) * float(np.float32(scale))
    raise ValueError(f"unknown KV format {kv_format!r}")


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Consecutive query heads share one KV head: with g = Hq/Hkv, heads [kvh*g, (kvh+1)*g)
    read KV head kvh."""
    return h // (num_q_heads // num_kv_heads)


def attended_range(L: int, window: int) -> Tuple[int, int]:
    """Token range [start, L) a decode query attends; window 0 means no window."""
    start = max(0, L - window) if window > 0 else 0
    return start, L


def gather_rows(cache: np.ndarray, block_table: np.ndarray, b: int, kvh: int,
                start: int, stop: int, block_size: int) -> np.ndarray:
    """Rows [start, stop) of sequence b, KV head kvh, as raw bf16 bits [stop-start][D].

    Token t is slot t % block_size of physical block block_table[b][t // block_size]."""
    t = np.arange(start, max(start, stop), dtype=np.int64)
    phys = block_table[b, t // block_size].astype(np.int64)
    return np.ascontiguousarray(cache[phys, kvh, t % block_size, :])


def softmax_attention(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                      sink: Optional[float] = None) -> Tuple[np.ndarray, float]:
    """out = softmax(scale * K q) V over the rows of K/V (float64), plus the natural-log LSE of
    the denominator.  A sink logit joins the max and the denominator with a zero value row."""
    D = V.shape[1] if V.ndim == 2 else qv.shape[0]
    logits = scale * (K @ qv) if K.shape[0] else np.zeros(0)
    parts = list(logits)
    if sink is not None:
        parts.append(float(sink))
    if not parts:
        return np.zeros(D), NEG_INF
    m = max(parts)
    w = np.exp(logits - m)
    Z = float(w.sum()) + (math.exp(float(sink) - m) if sink is not None else 0.0)
    out = (w @ V) / Z if K.shape[0] else np.zeros(D)
    return out, m + math.log(Z)


def decode_one(wl_q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
               block_table: np.ndarray, seq_lens: np.ndarray, scale: float, block_size: int,
               b: int, h: int, window: int = 0, sinks: Optional[np.ndarray] = None,
               num_kv_heads: Optional[int] = None, kv_format: str = "bf16",
               k_scale: float = 1.0, v_scale: float = 1.0) -> Tuple[np.ndarray, float]:
    """Output row and LSE of query head h of sequence b."""
    Hq = wl_q.shape[1]
    Hkv = k_cache.shape[1] if num_kv_heads is None else num_kv_heads
    kvh = kv_head_of(h, Hq, Hkv)
    start, stop = attended_range(int(seq_lens[b]), window)
    K = kv_rows_to_f64(gather_rows(k_cache, block_table, b, kvh, start, stop, block_size),
                       kv_format, k_scale)
    V = kv_rows_to_f64(gather_rows(v_cache, block_table, b, kvh, start, stop, block_size),
                       kv_format, v_scale)
    qv = bf16_bits_to_f64(wl_q[b, h])
    sink = None if sinks is None else float(np.float32(sinks[h]))
    return softmax_attention(qv, K, V, float(np.float32(scale)), sink)


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
           seq_lens: np.ndarray, scale: float, block_size: int, window: int = 0,
           sinks: Optional[np.ndarray] = None, kv_format: str = "bf16", k_scale: float = 1.0,
           v_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Whole batch: out float64 [B][Hq][D], lse float64 [B][Hq].  kv_format "bf16" (bit
    patterns) or "fp8_e4m3" (codes, with k_scale / v_scale)."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    sc = float(np.float32(scale))
    for b in range(B):
        start, stop = attended_range(int(seq_lens[b]), window)
        rows = {}
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            if kvh not in rows:
                rows[kvh] = (
                    kv_rows_to_f64(gather_rows(k_cache, block_table, b, kvh, start, stop,
                                               block_size), kv_format, k_scale),
                    kv_rows_to_f64(gather_rows(v_cache, block_table, b, kvh, start, stop,
                                               block_size), kv_format, v_scale))
            K, V = rows[kvh]
            sink = None if sinks is None else float(np.float32(sinks[h]))
            out[b, h], lse[b, h] = softmax_attention(bf16_bits_to_f64(q[b, h]), K, V, sc, sink)
    return out, lse


def query_range(L: int, q_len: int, i: int, window: int) -> Tuple[int, int]:
    """Keys [start, stop) that query token i of q_len attends in a sequence of length L (the new
    tokens included): causal up to its own position p = L - q_len + i, windowed to the last W
    keys up to p when W > 0.  Empty when p < 0."""
    p = L - q_len + i
    if p < 0:
        return 0, 0
    start = max(0, p + 1 - window) if window > 0 else 0
    return start, p + 1


def decode_multi(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_table: np.ndarray, seq_lens: np.ndarray, scale: float, block_size: int,
                 window: int = 0, sinks: Optional[np.ndarray] = None, kv_format: str = "bf16",
                 k_scale: float = 1.0, v_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """q_len query tokens per sequence: q bf16 bits [B][Q][Hq][D] -> out float64 [B][Q][Hq][D],
    lse float64 [B][Q][Hq].  Each (b, i, h) is the softmax attention of its query over the keys
    query_range gives, with the head's sink."""
    B, Q, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((B, Q, Hq, D))
    lse = np.full((B, Q, Hq), NEG_INF)
    sc = float(np.float32(scale))
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(Q):
            start, stop = query_range(L, Q, i, window)
            for h in range(Hq):
                kvh = kv_head_of(h, Hq, Hkv)
                K = kv_rows_to_f64(gather_rows(k_cache, block_table, b, kvh, start, stop,
                                               block_size), kv_format, k_scale)
                V = kv_rows_to_f64(gather_rows(v_cache, block_table, b, kvh, start, stop,
                                               block_size), kv_format, v_scale)
                sink = None if sinks is None else float(np.float32(sinks[h]))
                out[b, i, h], lse[b, i, h] = softmax_attention(bf16_bits_to_f64(q[b, i, h]), K,
                                                               V, sc, sink)
    return out, lse


def num_partitions(L: int, partition_size: int) -> int:
    """Partitions a sequence of length L occupies: at least one, so a sink on an empty sequence
    still has a partition to live in."""
    return max(1, -(-L // partition_size))


def decode_partitions(q, k_cache, v_cache, block_table, seq_lens, scale, block_size,
                      partition_size: int, max_partitions: Optional[int] = None, window: int = 0,
                      sinks: Optional[np.ndarray] = None):
    """Split-KV form: per partition p the softmax over [pP,(p+1)P) ∩ [start, L) alone.

    Returns o float64 [B][Hq][Pmax][D] (normalised within the partition) and lse float64
    [B][Hq][Pmax]; slots past a sequence's partition count hold o=0, lse=-inf."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    P = int(partition_size)
    if max_partitions is None:
        max_partitions = max(num_partitions(int(L), P) for L in seq_lens) if B else 1
    o = np.zeros((B, Hq, max_partitions, D))
    lse = np.full((B, Hq, max_partitions), NEG_INF)
    sc = float(np.float32(scale))
    for b in range(B):
        L = int(seq_lens[b])
        start, stop = attended_range(L, window)
        first = start // P
        for p in range(num_partitions(L, P)):
            lo, hi = max(start, p * P), min(stop, (p + 1) * P)
            rows = {}
            for h in range(Hq):
                kvh = kv_head_of(h, Hq, Hkv)
                if kvh not in rows:
                    rows[kvh] = (
                        bf16_bits_to_f64(gather_rows(k_cache, block_table, b, kvh, lo,
                                                     max(lo, hi), block_size)),
                        bf16_bits_to_f64(gather_rows(v_cache, block_table, b, kvh, lo,
                                                     max(lo, hi), block_size)))
                K, V = rows[kvh]
                sink = None
                if sinks is not None and p == first:
                    sink = float(np.float32(sinks[h]))
                o[b, h, p], lse[b, h, p] = softmax_attention(bf16_bits_to_f64(q[b, h]), K, V,
                                                             sc, sink)
    return o, lse


def merge_partitions(o: np.ndarray, lse: np.ndarray, counts: np.ndarray):
    """LSE-weighted merge of partials: for each (b, h) over its first counts[b] partitions,
    M = max lse_p, w_p = exp(lse_p - M), out = sum w_p o_p / sum w_p, lse = M + ln sum w_p.
    Partitions with lse = -inf carry no weight."""
    B, Hq, _, D = o.shape
    out = np.zeros((B, Hq, D))
    lse_out = np.full((B, Hq), NEG_INF)
    for b in range(B):
        n = int(counts[b])
        for h in range(Hq):
            ls = lse[b, h, :n]
            finite = np.isfinite(ls)
            if not finite.any():
                continue
            M = ls[finite].max()
            w = np.where(finite, np.exp(np.where(finite, ls, M) - M), 0.0)
            S = w.sum()
            acc = np.zeros(D)
            for p in range(n):
                if finite[p]:
                    acc += w[p] * o[b, h, p]
            out[b, h] = acc / S
            lse_out[b, h] = M + math.log(S)
    return out, lse_out

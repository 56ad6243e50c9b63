"""Seeded synthetic decode workloads shared by the tests, the bench and the oracle checks.

This module only *draws inputs*: sequence lengths, the physical-block permutation, the block
tables, and q/K/V/sink values.  It holds none of the attention arithmetic, so it is safe for both
the HIP path's tests and the oracle to consume the same bits.

Workload shapes follow the decode batches the pages measure (head_dim 128 GQA as in
Qwen3-dense/Llama/Mistral from vllm.cpp PR #564 "The gap it specs"; page-size-16 one-token
split-KV shapes from ROCm/rocm-libraries PR #13700 "Runnable saved-binding HIP-event
comparison").  All values are bf16 bit patterns (uint16) obtained from fp32 N(0,1) draws by
round-to-nearest-even.

Layouts (host, NumPy):
  q            uint16 [B][Hq][D]
  k_cache      uint16 [num_blocks][Hkv][block_size][D]
  v_cache      uint16 [num_blocks][Hkv][block_size][D]
  block_table  int32  [B][stride]      logical block i of sequence b -> physical block id
  seq_lens     int32  [B]
  sinks        float32 [Hq] or None
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BASE_SEED = 7
CHUNK = 1 << 22          # normals drawn per independently seeded chunk
BF16_QNAN = np.uint16(0x7FC0)

# stream ids inside one workload's SeedSequence
S_LENS, S_PERM, S_Q, S_K, S_V, S_SINKS = range(6)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _chunk_seed(root: np.random.SeedSequence, stream: int, chunk: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=root.entropy,
                                  spawn_key=tuple(root.spawn_key) + (stream, chunk))


def normal_bf16(root: np.random.SeedSequence, stream: int, n: int, mult: float = 1.0) -> np.ndarray:
    """n bf16 values ~ N(0,1)*mult, drawn in fixed, independently seeded chunks (thread-parallel,
    result independent of the thread count)."""
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(_chunk_seed(root, stream, c)))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


FP8_E4M3_MAX = 448.0
FP8_QNAN = np.uint8(0x7F)


def normal_fp8_e4m3(root: np.random.SeedSequence, stream: int, n: int, mult: float,
                    scale: float) -> np.ndarray:
    """n OCP FP8 E4M3 codes of N(0,1)*mult / scale: the same fp32 draws as normal_bf16, divided
    by the tensor scale, clipped to the format's range and rounded to nearest even by torch's
    float8_e4m3fn conversion."""
    import torch

    out = np.empty(n, dtype=np.uint8)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(_chunk_seed(root, stream, c)))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        x = np.clip(x / np.float32(scale), -FP8_E4M3_MAX, FP8_E4M3_MAX)
        out[lo:hi] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    for c in range(nchunks):
        fill(c)
    return out


def _rng(root: np.random.SeedSequence, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_chunk_seed(root, stream, 1 << 30)))


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seq_lens: np.ndarray            # int32 [B]
    block_table: np.ndarray         # int32 [B][stride]
    num_blocks: int
    q: np.ndarray                   # uint16 [B][Hq][D], or [B][q_len][Hq][D] when q_len > 1
    k_cache: np.ndarray             # [NB][Hkv][bs][D]: uint16 bf16 bits, or uint8 FP8 E4M3 codes
    v_cache: np.ndarray
    scale: np.float32
    window: int = 0
    sinks: Optional[np.ndarray] = None   # float32 [Hq]
    partition_size: int = 0
    meta: dict = field(default_factory=dict)
    kv_format: str = "bf16"         # "bf16" or "fp8_e4m3"
    k_scale: float = 1.0            # FP8: value = code value * scale
    v_scale: float = 1.0
    q_len: int = 1                  # new query tokens per sequence (the last q_len positions)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def window_span(self) -> int:
        """Keys before the last position that some query token can see: the union of the
        q_len queries' windows is W + q_len - 1 keys (0 = no window)."""
        return self.window + self.q_len - 1 if self.window > 0 else 0

    def attended_tokens(self) -> np.ndarray:
        """Tokens of each sequence that at least one query attends (their union)."""
        L = self.seq_lens.astype(np.int64)
        return np.minimum(L, self.window_span) if self.window > 0 else L

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step must read: every attended token's K and V row,
        once per KV head (2 bytes per value in bf16, 1 in FP8)."""
        elem = 1 if self.kv_format == "fp8_e4m3" else 2
        return int(self.attended_tokens().sum()) * self.num_kv_heads * self.head_dim * 2 * elem


def pool_blocks(seq_lens: Sequence[int], block_size: int, extra: float = 0.10) -> int:
    used = int(sum((int(L) + block_size - 1) // block_size for L in seq_lens))
    return int(math.ceil((1.0 + extra) * used)) if extra > 0 else used


def make_workload(*, name: str, seq_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                  head_dim: int, block_size: int, seed, num_blocks: Optional[int] = None,
                  window: int = 0, with_sinks: bool = False, k_mult: float = 1.0,
                  partition_size: int = 0, poison: bool = False, stride: Optional[int] = None,
                  scale: Optional[float] = None, unused_entry: str = "spare",
                  kv_format: str = "bf16", kv_scales=(1.0, 1.0), q_len: int = 1) -> Workload:
    """Build one seeded workload.

    Physical blocks are a seeded permutation of the pool; sequences take consecutive slices of it
    in batch order, logical order within each.  Unused block-table entries point at a spare
    (never attended) block, or hold -1 when ``unused_entry == "invalid"``.  With ``poison`` every
    K/V slot that no query attends (spare blocks, the tail slots of each last block, and the
    tokens before a sliding window) holds a bf16 NaN, so any stray read shows up in the output.
    With ``q_len`` > 1 there are q_len query tokens per sequence (q is [B][q_len][Hq][D]); the
    lengths count them, and the poison spares every key some query token attends.
    """
    root = np.random.SeedSequence(seed)
    L = np.asarray(seq_lens, dtype=np.int32)
    B = int(L.shape[0])
    bs = int(block_size)
    nblk = (L.astype(np.int64) + bs - 1) // bs
    used = int(nblk.sum())
    if num_blocks is None:
        num_blocks = pool_blocks(L, bs)
    if num_blocks < used + 1:
        num_blocks = used + 1   # keep one spare block for unused table entries
    if stride is None:
        stride = max(1, int(nblk.max()) if B else 1)
    perm = _rng(root, S_PERM).permutation(num_blocks).astype(np.int32)
    spare = int(perm[used])
    fill = -1 if unused_entry == "invalid" else spare
    bt = np.full((B, stride), fill, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    Hq, Hkv, D = int(num_q_heads), int(num_kv_heads), int(head_dim)
    Q = int(q_len)
    if Q < 1:
        raise ValueError("q_len must be at least 1")
    q = normal_bf16(root, S_Q, B * Q * Hq * D)
    q = q.reshape(B, Hq, D) if Q == 1 else q.reshape(B, Q, Hq, D)
    nkv = num_blocks * Hkv * bs * D
    if kv_format == "bf16":
        k = normal_bf16(root, S_K, nkv, k_mult).reshape(num_blocks, Hkv, bs, D)
        v = normal_bf16(root, S_V, nkv).reshape(num_blocks, Hkv, bs, D)
        nan = BF16_QNAN
    elif kv_format == "fp8_e4m3":
        k = normal_fp8_e4m3(root, S_K, nkv, k_mult, kv_scales[0]).reshape(num_blocks, Hkv, bs, D)
        v = normal_fp8_e4m3(root, S_V, nkv, 1.0, kv_scales[1]).reshape(num_blocks, Hkv, bs, D)
        nan = FP8_QNAN
    else:
        raise ValueError(f"unknown KV format {kv_format!r}")
    sinks = None
    if with_sinks:
        sinks = _rng(root, S_SINKS).standard_normal(Hq, dtype=np.float32)
    if poison:
        _poison(k, v, bt, L, bs, window + Q - 1 if window > 0 else 0, perm[used:], nan)
    sc = np.float32(1.0 / math.sqrt(D)) if scale is None else np.float32(scale)
    return Workload(name=name, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=bs, seq_lens=L, block_table=bt, num_blocks=int(num_blocks),
                    q=q, k_cache=k, v_cache=v, scale=sc, window=int(window), sinks=sinks,
                    partition_size=int(partition_size), meta={"seed": str(seed)},
                    kv_format=kv_format, k_scale=float(np.float32(kv_scales[0])),
                    v_scale=float(np.float32(kv_scales[1])), q_len=Q)


def _poison(k, v, bt, L, bs, window, spare_blocks, nan=BF16_QNAN) -> None:
    k[spare_blocks] = nan
    v[spare_blocks] = nan
    for b in range(bt.shape[0]):
        Lb = int(L[b])
        if Lb == 0:
            continue
        last = (Lb - 1) // bs
        tail = Lb - last * bs
        k[bt[b, last], :, tail:, :] = nan
        v[bt[b, last], :, tail:, :] = nan
        if window > 0 and Lb > window:
            start = Lb - window
            for i in range(start // bs + 1):
                lo = i * bs
                hi = min(start, lo + bs)
                k[bt[b, i], :, : hi - lo, :] = nan
                v[bt[b, i], :, : hi - lo, :] = nan


# ---------------------------------------------------------------------------------------------
# The five decode workloads (sizes as stated for this op; see the input recipe in the design doc)
# ---------------------------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny paged decode B2 L{37,100} 4q/2kv D128 bs16",
    2: "Llama-8B-shaped decode B64 L~U[512,4096] 32q/8kv D128 bs16",
    3: "head-size/GQA sweep B32 L8192 kv8 bs16",
    4: "long-context split-KV B4 L131072 64q/8kv D128 bs64 P512",
    5: "mixed batch window4096+sinks B128 L~lognormal(2048) 32q/8kv D128 bs16",
}

SWEEP_POINTS = [(D, hq) for D in (64, 128, 256) for hq in (8, 32, 64)]


def config_seq_lens(idx: int) -> np.ndarray:
    root = np.random.SeedSequence([BASE_SEED, idx])
    if idx == 1:
        return np.array([37, 100], dtype=np.int32)
    if idx == 2:
        return _rng(root, S_LENS).integers(512, 4096, size=64, endpoint=True).astype(np.int32)
    if idx == 3:
        return np.full(32, 8192, dtype=np.int32)
    if idx == 4:
        return np.full(4, 131072, dtype=np.int32)
    if idx == 5:
        z = _rng(root, S_LENS).standard_normal(128)
        Ls = np.rint(np.exp(math.log(2048.0) + z))
        return np.clip(Ls, 1, 32768).astype(np.int32)
    raise ValueError(f"no workload {idx}")


# FP8 KV variants: one fp32 scale per tensor (K, V); N(0,1) values divided by them stay well
# inside E4M3's +-448 range, and 0.05 is deliberately not a power of two
FP8_SCALES = (0.0625, 0.05)


def make_config(idx: int, *, head_dim: int = 128, num_q_heads: Optional[int] = None,
                poison: bool = False, seq_lens: Optional[Sequence[int]] = None,
                kv_format: str = "bf16", q_len: int = 1) -> Workload:
    """Workload ``idx`` in 1..5.  Workload 3 is a sweep: pick the point with ``head_dim`` in
    {64,128,256} and ``num_q_heads`` in {8,32,64} (8 KV heads).  ``kv_format="fp8_e4m3"`` gives
    the same workload with an FP8 E4M3 KV cache (scales FP8_SCALES)."""
    L = config_seq_lens(idx) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    name = CONFIG_NAMES[idx]
    kw = dict(poison=poison, kv_format=kv_format,
              kv_scales=FP8_SCALES if kv_format == "fp8_e4m3" else (1.0, 1.0), q_len=q_len)
    if kv_format != "bf16":
        name = f"{name} kv={kv_format}"
    if q_len > 1:
        name = f"{name} q_len={q_len}"
    if idx == 1:
        return make_workload(name=name, seq_lens=L, num_q_heads=4, num_kv_heads=2, head_dim=128,
                             block_size=16, num_blocks=32, seed=[BASE_SEED, 1], **kw)
    if idx == 2:
        return make_workload(name=name, seq_lens=L, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, seed=[BASE_SEED, 2], **kw)
    if idx == 3:
        hq = 32 if num_q_heads is None else int(num_q_heads)
        return make_workload(name=f"{name} D{head_dim} {hq}q", seq_lens=L, num_q_heads=hq,
                             num_kv_heads=8, head_dim=head_dim, block_size=16,
                             seed=[BASE_SEED, 3, head_dim, hq], **kw)
    if idx == 4:
        return make_workload(name=name, seq_lens=L, num_q_heads=64, num_kv_heads=8, head_dim=128,
                             block_size=64, seed=[BASE_SEED, 4], k_mult=0.5, partition_size=512,
                             **kw)
    if idx == 5:
        return make_workload(name=name, seq_lens=L, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, seed=[BASE_SEED, 5], window=4096, with_sinks=True,
                             **kw)
    raise ValueError(f"no workload {idx}")

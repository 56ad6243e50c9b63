"""Test and measurement entry points (include/paged_attn_debug.h): the gather witnesses, the
streaming-read and gather-read probes, the plain copy kernel and a plan run with the decode
kernel bracketed by HIP events.  Argument marshalling only."""
from __future__ import annotations

import ctypes

import torch

from . import (KV_DTYPES, PA_OK, PagedAttnError, _BF16_LIKE, _dev, _layout_ptr, _ptr, _stream,
               lib, make_shape)


def gather_witness(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, *, num_seqs: int, window: int = 0, max_rows: int,
                   stream=None):
    """Rows the decode kernels' address generator selects: bf16 bits as int16
    [B][Hkv][max_rows][D] for K and V (unwritten rows keep the bits 0xFFFF)."""
    _dev(k_cache, "k_cache", _BF16_LIKE)
    _dev(v_cache, "v_cache", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    NB, Hkv, bs, D = k_cache.shape
    k_rows = torch.full((num_seqs, Hkv, max_rows, D), -1, dtype=torch.int16,
                        device=k_cache.device)
    v_rows = k_rows.clone()
    shape = make_shape(num_seqs, Hkv, Hkv, NB, block_table.shape[1])
    st = lib().paged_attn_gather_witness(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(block_table), _ptr(seq_lens), int(D), int(bs),
                                         int(window), int(max_rows), _ptr(k_rows), _ptr(v_rows),
                                         _stream(k_cache.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_gather_witness")
    return k_rows, v_rows


def gather_witness_balanced(k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor, *, num_seqs: int,
                            num_kv_heads: int, num_blocks: int, head_dim: int, block_size: int,
                            num_workers: int, max_rows: int, window: int = 0,
                            kv_dtype: str = "bf16", kv_layout=None, stream=None):
    """Rows the balanced decode kernel's walk selects with ``num_workers`` workers: uint8
    [B][Hkv][max_rows][row bytes] for K and V (unwritten rows keep 0xEE bytes).  The pools may
    be in any layout given by ``kv_layout`` strides (elements), as for Plan."""
    _dev(block_table, "block_table", (torch.int32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    if not (k_cache.is_cuda and v_cache.is_cuda):
        raise ValueError("k_cache and v_cache must be GPU tensors")
    row = head_dim * (1 if kv_dtype == "fp8_e4m3" else 2)
    k_rows = torch.full((num_seqs, num_kv_heads, max_rows, row), 0xEE, dtype=torch.uint8,
                        device=k_cache.device)
    v_rows = k_rows.clone()
    shape = make_shape(num_seqs, num_kv_heads, num_kv_heads, num_blocks, block_table.shape[1])
    st = lib().paged_attn_gather_witness_balanced(
        ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        int(head_dim), int(block_size), int(window), KV_DTYPES[kv_dtype], _layout_ptr(kv_layout),
        int(num_workers), int(max_rows), _ptr(k_rows), _ptr(v_rows),
        _stream(k_cache.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_gather_witness_balanced")
    return k_rows, v_rows


def stream_read(buf: torch.Tensor, num_workgroups: int, sink: torch.Tensor, stream=None) -> None:
    nbytes = buf.numel() * buf.element_size()
    st = lib().paged_attn_stream_read(_ptr(buf), nbytes, int(num_workgroups), _ptr(sink),
                                      _stream(buf.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_stream_read")


def gather_read(buf: torch.Tensor, chunk_bytes: int, chunk_ids: torch.Tensor,
                num_workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """Read the chunks of `buf` listed in chunk_ids (int32, device) in that order."""
    _dev(chunk_ids, "chunk_ids", (torch.int32,))
    nbytes = buf.numel() * buf.element_size()
    st = lib().paged_attn_gather_read(_ptr(buf), nbytes, int(chunk_bytes), _ptr(chunk_ids),
                                      int(chunk_ids.numel()), int(num_workgroups), _ptr(sink),
                                      _stream(buf.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_gather_read")


def copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    st = lib().paged_attn_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_copy")


def plan_run_timed(plan, q, k_cache, v_cache, block_table, seq_lens, scale: float, *, out,
                   ev_before, ev_after, lse=None, sinks=None, workspace=None, stream=None,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Plan.run with ``ev_before`` / ``ev_after`` (torch.cuda.Event objects, already created:
    record each once before the first call) recorded on the launch stream right before and
    after the plan's decode kernel, so that ``ev_before.elapsed_time(ev_after)`` is that
    kernel's own duration."""
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("out", out),
                    ("lse", lse), ("sinks", sinks), ("workspace", workspace)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    h0, h1 = ev_before.cuda_event, ev_after.cuda_event
    if not h0 or not h1:
        raise ValueError("record the events once before passing them")
    st = lib().paged_attn_plan_run_timed(plan._h, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(block_table), _ptr(seq_lens), float(scale),
                                         float(k_scale), float(v_scale), _ptr(sinks), _ptr(out),
                                         _ptr(lse), _ptr(workspace),
                                         _stream(out.device, stream), h0, h1)
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_plan_run_timed")

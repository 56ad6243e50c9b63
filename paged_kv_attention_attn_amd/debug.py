"""Test and measurement entry points (include/paged_attn_debug.h): the gather witness, the
streaming-read probe and the plain copy kernel.  Argument marshalling only."""
from __future__ import annotations

import ctypes

import torch

from . import PA_OK, PagedAttnError, _dev, _ptr, _stream, _BF16_LIKE, lib, make_shape


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


def stream_read(buf: torch.Tensor, num_workgroups: int, sink: torch.Tensor, stream=None) -> None:
    nbytes = buf.numel() * buf.element_size()
    st = lib().paged_attn_stream_read(_ptr(buf), nbytes, int(num_workgroups), _ptr(sink),
                                      _stream(buf.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_stream_read")


def copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    st = lib().paged_attn_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_copy")

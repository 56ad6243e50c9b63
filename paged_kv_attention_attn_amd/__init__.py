"""Python binding of the gfx950 paged-attention decode library (libpaged_attn.so).

Argument marshalling only: every step of the decode runs in the HIP kernels behind the C ABI
declared in include/paged_attn.h.  PyTorch provides device memory and the current stream.  If
the library has not been built, importing this package raises; there is no fallback path.

    from paged_kv_attention_attn_amd import decode, reduce
    out, lse = decode(q, k_cache, v_cache, block_table, seq_lens, scale)          # unsplit
    part, plse = decode(..., partition_size=512, max_partitions=256)              # split
    out, lse = reduce(part, plse, seq_lens, partition_size=512)

Tensor layouts (all on the GPU, contiguous): q bf16 [B][Hq][D]; k_cache / v_cache bf16
[num_blocks][Hkv][block_size][D]; block_table int32 [B][stride]; seq_lens int32 [B];
sinks fp32 [Hq]; out fp32 [B][Hq][D] (split: [B][Hq][max_partitions][D]); lse fp32 [B][Hq]
(split: [B][Hq][max_partitions]).  bf16 tensors may also be passed as uint16/int16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; PA_LIBRARY names another build of the same sources to load instead (the
# sanitizer build of the host code that a CPU test runs the ABI tests against).
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpaged_attn.so")

PA_OK = 0
STATUS_NAMES = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
                -4: "PA_ERR_LSE_REQUIRED", -5: "PA_ERR_LAUNCH", -6: "PA_ERR_TABLE"}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


class PaShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_table_stride", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("max_partitions", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python paged_kv_attention_attn_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    sp = ctypes.POINTER(PaShape)
    sigs = {
        "paged_attn_decode": (i32, [sp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp, vp, vp]),
        "paged_attn_reduce": (i32, [sp, i32, vp, vp, vp, vp, vp, vp]),
        "paged_attn_num_partitions": (i32, [i32, i32]),
        "paged_attn_variant_name": (ctypes.c_char_p, [sp, i32, i32]),
        "paged_attn_status_string": (ctypes.c_char_p, [i32]),
        "paged_attn_check_tables": (i32, [sp, i32, i32, vp, vp]),
        "paged_attn_suggest_partition_size": (i32, [i32, i32, i32, i32, i32]),
        "paged_attn_suggest_schedule": (i32, [i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(i32)]),
        "paged_attn_abi_version": (i32, []),
        "paged_attn_decode_balanced": (i32, [sp, vp, vp, vp, vp, vp, f32, i32, i32, i32, vp, vp,
                                             vp, vp, ctypes.c_size_t, i32, vp]),
        "paged_attn_reduce_balanced": (i32, [sp, vp, i32, i32, i32, vp, vp, vp, vp,
                                             ctypes.c_size_t, i32, vp]),
        "paged_attn_decode_balanced_noalloc": (i32, [sp, vp, vp, vp, vp, vp, f32, i32, i32, i32,
                                                     vp, vp, vp, i32, vp]),
        "paged_attn_balanced_workspace_size": (ctypes.c_int64, [sp, i32, i32]),
        "paged_attn_balanced_default_workers": (i32, [i32, i32]),
        "paged_attn_plan_create": (i32, [sp, i32, i32, i32, i32, i32, vp, i32, i32, i32,
                                         ctypes.POINTER(vp)]),
        "paged_attn_plan_create_flags": (i32, [sp, i32, i32, i32, i32, i32, vp, i32, i32, i32,
                                               i32, ctypes.POINTER(vp)]),
        "paged_attn_plan_workspace_size": (ctypes.c_int64, [vp]),
        "paged_attn_plan_run": (i32, [vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, vp, vp,
                                      vp]),
        "paged_attn_plan_run_timed": (i32, [vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, vp,
                                            vp, vp, vp, vp]),
        "paged_attn_plan_name": (ctypes.c_char_p, [vp]),
        "paged_attn_plan_destroy": (None, [vp]),
        "paged_attn_gather_witness": (i32, [sp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]),
        "paged_attn_gather_witness_balanced": (i32, [sp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                     i32, i32, vp, vp, vp]),
        "paged_attn_stream_read": (i32, [vp, ctypes.c_size_t, i32, vp, vp]),
        "paged_attn_gather_read": (i32, [vp, ctypes.c_size_t, i32, vp, ctypes.c_int64, i32, vp,
                                         vp]),
        "paged_attn_copy": (i32, [vp, vp, ctypes.c_size_t, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("paged_attn_decode", "paged_attn_reduce", "paged_attn_decode_balanced",
            "paged_attn_reduce_balanced", "paged_attn_decode_balanced_noalloc",
            "paged_attn_balanced_workspace_size", "paged_attn_balanced_default_workers",
            "paged_attn_num_partitions",
            "paged_attn_variant_name", "paged_attn_status_string", "paged_attn_check_tables",
            "paged_attn_suggest_partition_size", "paged_attn_suggest_schedule",
            "paged_attn_abi_version",
            "paged_attn_gather_witness", "paged_attn_gather_witness_balanced",
            "paged_attn_stream_read", "paged_attn_gather_read",
            "paged_attn_copy",
            "paged_attn_plan_create", "paged_attn_plan_create_flags",
            "paged_attn_plan_workspace_size", "paged_attn_plan_run",
            "paged_attn_plan_run_timed", "paged_attn_plan_name", "paged_attn_plan_destroy")


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.paged_attn_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.paged_attn_abi_version())


def num_partitions(seq_len: int, partition_size: int) -> int:
    return int(_lib.paged_attn_num_partitions(int(seq_len), int(partition_size)))


def suggest_partition_size(num_seqs: int, num_kv_heads: int, max_seq_len: int, block_size: int,
                           num_cus: int) -> int:
    return int(_lib.paged_attn_suggest_partition_size(num_seqs, num_kv_heads, max_seq_len,
                                                      block_size, num_cus))


def suggest_schedule(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     block_size: int, *, window: int = 0, q_len: int = 1, max_seq_len: int = 0,
                     num_cus: int = 0) -> Tuple[str, int]:
    """(schedule name, partition_size) the library suggests for a plan of these sizes
    (paged_attn_suggest_schedule; num_cus 0 = the current device's)."""
    P = ctypes.c_int32(0)
    r = int(_lib.paged_attn_suggest_schedule(int(num_seqs), int(num_q_heads), int(num_kv_heads),
                                             int(head_dim), int(block_size), int(window),
                                             int(q_len), int(max_seq_len), int(num_cus),
                                             ctypes.byref(P)))
    if r < 0:
        raise PagedAttnError(r, "paged_attn_suggest_schedule")
    return {v: k for k, v in SCHEDULES.items()}[r], int(P.value)


def make_shape(num_seqs: int, num_q_heads: int, num_kv_heads: int, num_blocks: int,
               block_table_stride: int, partition_size: int = 0,
               max_partitions: int = 0) -> PaShape:
    return PaShape(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(num_blocks),
                   int(block_table_stride), int(partition_size), int(max_partitions))


def variant_name(shape: PaShape, head_dim: int, block_size: int) -> Optional[str]:
    r = _lib.paged_attn_variant_name(ctypes.byref(shape), int(head_dim), int(block_size))
    return None if r is None else r.decode()


def check_tables(shape: PaShape, block_size: int, window: int, block_table_host,
                 seq_lens_host) -> int:
    """Host-side table check on CPU int32 tensors / NumPy arrays; returns the status code."""
    bt = torch.as_tensor(block_table_host, dtype=torch.int32).contiguous()
    sl = torch.as_tensor(seq_lens_host, dtype=torch.int32).contiguous()
    return int(_lib.paged_attn_check_tables(ctypes.byref(shape), int(block_size), int(window),
                                            ctypes.c_void_p(bt.data_ptr()),
                                            ctypes.c_void_p(sl.data_ptr())))


# ---------------------------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------------------------
_BF16_LIKE = (torch.bfloat16, torch.uint16, torch.int16)


def _dev(t: torch.Tensor, name: str, dtypes) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, *, window: int = 0,
           sinks: Optional[torch.Tensor] = None, partition_size: int = 0,
           max_partitions: Optional[int] = None, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, want_lse: bool = True,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """paged_attn_decode on torch tensors.  Unsplit: returns (out [B][Hq][D], lse [B][Hq] or
    None).  Split (partition_size > 0): returns the partials ([B][Hq][Pmax][D], [B][Hq][Pmax]);
    max_partitions must be given (or implied by ``out``)."""
    _dev(q, "q", _BF16_LIKE)
    _dev(k_cache, "k_cache", _BF16_LIKE)
    _dev(v_cache, "v_cache", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B][Hq][D]; k_cache/v_cache [num_blocks][Hkv][bs][D], equal")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("inconsistent q / cache / block_table / seq_lens shapes")
    split = partition_size > 0
    if split:
        if max_partitions is None:
            if out is None:
                raise ValueError("split mode needs max_partitions (or an out tensor)")
            max_partitions = out.shape[2]
    else:
        max_partitions = 0
    if sinks is not None:
        _dev(sinks, "sinks", (torch.float32,))
        if sinks.shape != (Hq,):
            raise ValueError("sinks must be fp32 [Hq]")
    if out is None:
        shp = (B, Hq, max_partitions, D) if split else (B, Hq, D)
        out = torch.empty(shp, dtype=torch.float32, device=q.device)
    else:
        _dev(out, "out", (torch.float32,))
    if lse is None and (split or want_lse):
        shp = (B, Hq, max_partitions) if split else (B, Hq)
        lse = torch.empty(shp, dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", (torch.float32,))
    shape = make_shape(B, Hq, Hkv, NB, block_table.shape[1], partition_size, max_partitions)
    st = _lib.paged_attn_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_table), _ptr(seq_lens), float(scale), int(D),
                                int(bs), int(window), _ptr(sinks), _ptr(out), _ptr(lse),
                                _stream(q.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_decode")
    return out, lse


def reduce(partials: torch.Tensor, lse_partials: torch.Tensor, seq_lens: torch.Tensor, *,
           partition_size: int, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, want_lse: bool = True,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """paged_attn_reduce on torch tensors: merges [B][Hq][Pmax][D] partials into [B][Hq][D]."""
    _dev(partials, "partials", (torch.float32,))
    _dev(lse_partials, "lse_partials", (torch.float32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    B, Hq, Pmax, D = partials.shape
    if lse_partials.shape != (B, Hq, Pmax) or seq_lens.shape != (B,):
        raise ValueError("inconsistent partial / lse / seq_lens shapes")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=partials.device)
    else:
        _dev(out, "out", (torch.float32,))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=partials.device)
    elif lse is not None:
        _dev(lse, "lse", (torch.float32,))
    # the reducer reads only the sizes below from the shape
    shape = make_shape(B, Hq, 1, 1, 1, partition_size, Pmax)
    st = _lib.paged_attn_reduce(ctypes.byref(shape), int(D), _ptr(partials), _ptr(lse_partials),
                                _ptr(seq_lens), _ptr(out), _ptr(lse),
                                _stream(partials.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_reduce")
    return out, lse


def balanced_default_workers(head_dim: int, group: int) -> int:
    n = int(_lib.paged_attn_balanced_default_workers(int(head_dim), int(group)))
    if n <= 0:
        raise PagedAttnError(n, "paged_attn_balanced_default_workers")
    return n


def decode_balanced_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, *,
                            out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                            window: int = 0, sinks: Optional[torch.Tensor] = None,
                            num_workers: int = 0, stream=None) -> None:
    """paged_attn_decode_balanced_noalloc: the balanced step (decode + merge) into the caller's
    out (fp32 [B][Hq][D]) and lse (fp32 [B][Hq] or None) with the library's own device array for
    the partials; allocates nothing."""
    _dev(q, "q", _BF16_LIKE)
    _dev(k_cache, "k_cache", _BF16_LIKE)
    _dev(v_cache, "v_cache", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    _dev(out, "out", (torch.float32,))
    if lse is not None:
        _dev(lse, "lse", (torch.float32,))
    if sinks is not None:
        _dev(sinks, "sinks", (torch.float32,))
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B][Hq][D]; k_cache/v_cache [num_blocks][Hkv][bs][D], equal")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,) \
            or out.shape != (B, Hq, D) or (lse is not None and lse.shape != (B, Hq)) \
            or (sinks is not None and sinks.shape != (Hq,)):
        raise ValueError("inconsistent q / cache / block_table / seq_lens / out / lse / sinks")
    shape = make_shape(B, Hq, Hkv, NB, block_table.shape[1])
    st = _lib.paged_attn_decode_balanced_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), float(scale), int(D), int(bs), int(window), _ptr(sinks), _ptr(out),
        _ptr(lse), int(num_workers), _stream(q.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_decode_balanced_noalloc")


def balanced_workspace_size(shape: PaShape, head_dim: int, num_workers: int = 0) -> int:
    n = int(_lib.paged_attn_balanced_workspace_size(ctypes.byref(shape), int(head_dim),
                                                    int(num_workers)))
    if n < 0:
        raise PagedAttnError(n, "paged_attn_balanced_workspace_size")
    return n


def decode_balanced(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, *,
                    window: int = 0, sinks: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    want_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                    num_workers: int = 0, merge: bool = True, stream=None):
    """paged_attn_decode_balanced (+ paged_attn_reduce_balanced when ``merge``) on torch tensors:
    the final (out [B][Hq][D], lse [B][Hq] or None).  ``workspace`` (a device tensor of at least
    balanced_workspace_size bytes) is allocated here when not given; with merge=False the caller
    runs reduce_balanced with the same arguments and workspace."""
    _dev(q, "q", _BF16_LIKE)
    _dev(k_cache, "k_cache", _BF16_LIKE)
    _dev(v_cache, "v_cache", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B][Hq][D]; k_cache/v_cache [num_blocks][Hkv][bs][D], equal")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("inconsistent q / cache / block_table / seq_lens shapes")
    if sinks is not None:
        _dev(sinks, "sinks", (torch.float32,))
        if sinks.shape != (Hq,):
            raise ValueError("sinks must be fp32 [Hq]")
    shape = make_shape(B, Hq, Hkv, NB, block_table.shape[1])
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    else:
        _dev(out, "out", (torch.float32,))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", (torch.float32,))
    need = balanced_workspace_size(shape, D, num_workers)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.paged_attn_decode_balanced(ctypes.byref(shape), _ptr(q), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                         float(scale), int(D), int(bs), int(window),
                                         _ptr(sinks), _ptr(out), _ptr(lse), _ptr(workspace),
                                         nbytes, int(num_workers), _stream(q.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_decode_balanced")
    if merge:
        reduce_balanced(seq_lens, out, lse, shape=shape, head_dim=D, block_size=bs,
                        window=window, sinks=sinks, workspace=workspace, num_workers=num_workers,
                        stream=stream)
    return out, lse


def reduce_balanced(seq_lens: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor], *,
                    shape: PaShape, head_dim: int, block_size: int, window: int = 0,
                    sinks: Optional[torch.Tensor] = None, workspace: torch.Tensor,
                    num_workers: int = 0, stream=None) -> None:
    """paged_attn_reduce_balanced: merge the partials decode_balanced left in ``workspace``."""
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.paged_attn_reduce_balanced(ctypes.byref(shape), _ptr(seq_lens), int(head_dim),
                                         int(block_size), int(window), _ptr(sinks), _ptr(out),
                                         _ptr(lse), _ptr(workspace), nbytes, int(num_workers),
                                         _stream(out.device, stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attn_reduce_balanced")


def paged_attention(q, k_cache, v_cache, block_table, seq_lens, scale, *, window: int = 0,
                    sinks=None, partition_size: int = 0, max_seq_len: Optional[int] = None,
                    want_lse: bool = True, stream=None):
    """One decode step end to end: decode (+ reduce when partition_size > 0).  In split mode
    ``max_seq_len`` (a host-side bound on seq_lens) sizes the partial buffers.
    partition_size = -1 selects the balanced schedule (decode_balanced)."""
    if partition_size < 0:
        return decode_balanced(q, k_cache, v_cache, block_table, seq_lens, scale, window=window,
                               sinks=sinks, want_lse=want_lse, stream=stream)
    if partition_size == 0:
        return decode(q, k_cache, v_cache, block_table, seq_lens, scale, window=window,
                      sinks=sinks, want_lse=want_lse, stream=stream)
    if max_seq_len is None:
        raise ValueError("split mode needs max_seq_len")
    pmax = num_partitions(int(max_seq_len), int(partition_size))
    part, plse = decode(q, k_cache, v_cache, block_table, seq_lens, scale, window=window,
                        sinks=sinks, partition_size=partition_size, max_partitions=pmax,
                        stream=stream)
    return reduce(part, plse, seq_lens, partition_size=partition_size, want_lse=want_lse,
                  stream=stream)


SCHEDULES = {"unsplit": 0, "partitioned": 1, "balanced": 2, "fused": 3, "query_blocks": 4}


class KvLayout(ctypes.Structure):
    """pa_kv_layout: row (block, head, slot) at block*block_stride + head*head_stride +
    slot*token_stride elements."""
    _fields_ = [("block_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64)]


def _layout_ptr(layout):
    if layout is None:
        return None
    return ctypes.cast(ctypes.pointer(KvLayout(*[int(x) for x in layout])), ctypes.c_void_p)
KV_DTYPES = {"bf16": 0, "fp8_e4m3": 1}
PLAN_P_ONE_BF16 = 1   # PA_PLAN_P_ONE_BF16


class Plan:
    """A prepared decode step (paged_attn_plan_*): checks, variant choice and launch geometry
    done once; run() fills pointers and launches decode (+ merge).  ``schedule`` is "unsplit",
    "partitioned" (``partition_size`` tokens, partition slots for ``max_seq_len``), "fused"
    (partitioned, merged in the same launch by the last partition to finish), "balanced"
    (``num_workers``, 0 = the device default; ``max_seq_len``, a bound on the lengths, caps the
    workers of a small batch) or "query_blocks" (several query tokens: one wave per (sequence,
    KV head, block of tokens); with ``max_seq_len`` given and too few blocks to fill the GPU,
    key splits merged by a second kernel, which take a workspace), or "auto": the schedule and
    partition size suggest_schedule() gives for these sizes on the current device (the chosen
    one is in ``schedule``).  ``kv_dtype`` is "bf16" or "fp8_e4m3" (KV pools
    of one byte per value, uint8 tensors, with per-tensor scales given to run()).
    ``kv_layout``: None for the pool [num_blocks][Hkv][bs][D], else (block, head, token) strides
    in elements of the cache type (pa_kv_layout).
    ``q_len`` > 1 (balanced or query_blocks): q_len causal query tokens per sequence,
    q [B][q_len][Hq][D] -> out [B][q_len][Hq][D], lse [B][q_len][Hq].  ``p_terms``: 2 (the
    default) forms P.V with P as two bf16 terms; 1 rounds P to one bf16 term where the query-block
    schedule's 32-key form runs (PA_PLAN_P_ONE_BF16: faster, outputs within 2^-8 max|v| of the
    two-term result; the name then ends in "_p1").  run() records only kernel launches on the
    stream, so it can be captured in a CUDA/HIP graph."""

    def __init__(self, num_seqs: int, num_q_heads: int, num_kv_heads: int, num_blocks: int,
                 block_table_stride: int, head_dim: int, block_size: int, *, window: int = 0,
                 schedule: str = "balanced", partition_size: int = 0,
                 max_seq_len: Optional[int] = None, num_workers: int = 0,
                 kv_dtype: str = "bf16", q_len: int = 1,
                 kv_layout: Optional[Tuple[int, int, int]] = None, p_terms: int = 2):
        if schedule == "auto":
            schedule, partition_size = suggest_schedule(
                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, window=window,
                q_len=q_len, max_seq_len=max_seq_len or 0)
        if schedule not in SCHEDULES:
            raise ValueError(f"schedule must be 'auto' or one of {sorted(SCHEDULES)}")
        self.schedule = schedule
        if kv_dtype not in KV_DTYPES:
            raise ValueError(f"kv_dtype must be one of {sorted(KV_DTYPES)}")
        self.kv_dtype = kv_dtype
        pmax = 0
        if schedule in ("partitioned", "fused"):
            if partition_size <= 0 or max_seq_len is None:
                raise ValueError(f"the {schedule} schedule needs partition_size and "
                                 "max_seq_len")
            pmax = num_partitions(int(max_seq_len), int(partition_size))
        else:
            partition_size = 0
        self.shape = make_shape(num_seqs, num_q_heads, num_kv_heads, num_blocks,
                                block_table_stride, partition_size, pmax)
        self.dims = (num_seqs, num_q_heads, head_dim)
        self._h = ctypes.c_void_p()
        if p_terms not in (1, 2):
            raise ValueError("p_terms must be 1 or 2")
        st = _lib.paged_attn_plan_create_flags(
            ctypes.byref(self.shape), int(head_dim), int(block_size), int(window),
            SCHEDULES[schedule], KV_DTYPES[kv_dtype], _layout_ptr(kv_layout), int(q_len),
            int(max_seq_len or 0), int(num_workers), PLAN_P_ONE_BF16 if p_terms == 1 else 0,
            ctypes.byref(self._h))
        if st != PA_OK:
            raise PagedAttnError(st, "paged_attn_plan_create")
        self.workspace_size = int(_lib.paged_attn_plan_workspace_size(self._h))
        self.name = _lib.paged_attn_plan_name(self._h).decode()

    def workspace(self, device) -> Optional[torch.Tensor]:
        """A zero-filled workspace tensor of the size the plan needs (None when it needs
        none)."""
        if self.workspace_size == 0:
            return None
        return torch.zeros(self.workspace_size, dtype=torch.uint8, device=device)

    def run(self, q, k_cache, v_cache, block_table, seq_lens, scale: float, *, out, lse=None,
            sinks=None, workspace=None, stream=None, k_scale: float = 1.0,
            v_scale: float = 1.0) -> None:
        """One step into the caller's ``out`` (fp32 [B][Hq][D]) and ``lse`` (fp32 [B][Hq] or
        None).  ``k_scale`` / ``v_scale``: an FP8 cache's per-tensor scales (1 for bf16).
        Pointers only: the tensors must match the sizes the plan was made for (only their being
        on the GPU is checked here)."""
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                        ("block_table", block_table), ("seq_lens", seq_lens), ("out", out),
                        ("lse", lse), ("sinks", sinks), ("workspace", workspace)):
            if t is not None and not t.is_cuda:
                raise ValueError(f"{name} must be a GPU tensor")
        st = _lib.paged_attn_plan_run(self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(block_table), _ptr(seq_lens), float(scale),
                                      float(k_scale), float(v_scale),
                                      _ptr(sinks), _ptr(out), _ptr(lse), _ptr(workspace),
                                      _stream(out.device, stream))
        if st != PA_OK:
            raise PagedAttnError(st, "paged_attn_plan_run")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib.paged_attn_plan_destroy(h)
            self._h = ctypes.c_void_p()

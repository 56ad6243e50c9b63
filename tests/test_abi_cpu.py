"""C-ABI tests that need no GPU: the library loads, exports every declared symbol, and rejects
bad descriptors on the host before any launch (no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    names = set()
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(paged_attn_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "paged_attn_decode" in names and "paged_attn_reduce" in names
    lib = ctypes.CDLL(pa.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(pa.EXPORTED) == names


def test_abi_version_and_status_strings():
    assert pa.abi_version() == 5
    for code, name in pa.STATUS_NAMES.items():
        s = pa.status_string(code)
        assert s and s != "unknown status", name
    assert pa.status_string(12345) == "unknown status"


@pytest.mark.parametrize("L,P,n", [(0, 0, 1), (5, 0, 1), (0, 512, 1), (1, 512, 1), (512, 512, 1),
                                   (513, 512, 2), (131072, 512, 256), (-1, 16, -1), (3, -16, -1)])
def test_num_partitions(L, P, n):
    assert pa.num_partitions(L, P) == n


def shape(**kw):
    d = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, num_blocks=32, block_table_stride=8,
             partition_size=0, max_partitions=0)
    d.update(kw)
    return pa.make_shape(**d)


def test_variant_names(monkeypatch):
    monkeypatch.delenv("PA_DECODE_PATH", raising=False)
    monkeypatch.delenv("PA_DECODE_WAVES", raising=False)
    # default score path: P.V on the matrix cores from two query heads per KV head up
    assert pa.variant_name(shape(), 128, 16) == "pa_decode_mfmapv_d128_g4_w4"
    assert pa.variant_name(shape(num_q_heads=2), 128, 16) == "pa_decode_mfma_d128_g1_w4"
    monkeypatch.setenv("PA_DECODE_PATH", "mfma_pv")
    assert pa.variant_name(shape(num_q_heads=2), 64, 16) == "pa_decode_mfmapv_d64_g1_w4"
    monkeypatch.setenv("PA_DECODE_PATH", "mfma")
    monkeypatch.setenv("PA_DECODE_WAVES", "4")
    assert pa.variant_name(shape(), 128, 16) == "pa_decode_mfma_d128_g4_w4"
    assert pa.variant_name(shape(partition_size=512, max_partitions=4), 64, 64) == \
        "pa_decode_mfma_d64_g4_w4_split"
    monkeypatch.setenv("PA_DECODE_PATH", "valu")
    monkeypatch.setenv("PA_DECODE_WAVES", "2")
    assert pa.variant_name(shape(), 256, 16) == "pa_decode_valu_d256_g4_w2"
    assert pa.variant_name(shape(num_q_heads=6, num_kv_heads=2), 128, 16) is None   # g = 3
    assert pa.variant_name(shape(), 96, 16) is None
    assert pa.variant_name(shape(), 128, 8) is None


def call_decode(s, *, head_dim=128, block_size=16, window=0, scale=0.1, q=FAKE, out=FAKE,
                lse=None, sinks=None, shape_ptr=True):
    sp = ctypes.byref(s) if shape_ptr else None
    return pa.lib().paged_attn_decode(sp, q, FAKE, FAKE, FAKE, FAKE, scale, head_dim, block_size,
                                      window, sinks, out, lse, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(shape_ptr=False), -1),
    (dict(head_dim=96), -3), (dict(head_dim=512), -3),
    (dict(block_size=8), -3), (dict(block_size=48), -3), (dict(block_size=512), -3),
    (dict(window=-1), -2), (dict(scale=float("nan")), -2), (dict(scale=float("inf")), -2),
    (dict(q=None), -1), (dict(out=None), -1),
])
def test_decode_rejects(kw, expect):
    assert call_decode(shape(), **kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(num_q_heads=6, num_kv_heads=4), -2),          # Hq % Hkv != 0
    (dict(num_q_heads=6, num_kv_heads=2), -3),          # g = 3 not compiled
    (dict(num_q_heads=32, num_kv_heads=2), -3),         # g = 16 not compiled
    (dict(num_seqs=-1), -2), (dict(num_q_heads=0), -2), (dict(num_kv_heads=0), -2),
    (dict(num_blocks=0), -2), (dict(block_table_stride=0), -2),
    (dict(partition_size=-16), -2),
    (dict(partition_size=40, max_partitions=4), -2),    # not a multiple of 16
    (dict(partition_size=512, max_partitions=0), -2),
    (dict(partition_size=512, max_partitions=4), -4),   # split without lse
    (dict(num_seqs=70000), -2),                         # grid limit
])
def test_decode_rejects_shape(kw, expect):
    assert call_decode(shape(**kw)) == expect


@pytest.mark.parametrize("var,val", [("PA_DECODE_PATH", "VALU"), ("PA_DECODE_PATH", "auto"),
                                     ("PA_DECODE_PATH", "mfmapv"), ("PA_DECODE_PATH", "mfma_pv "),
                                     ("PA_DECODE_WAVES", "3"), ("PA_DECODE_WAVES", "4 "),
                                     ("PA_DECODE_WAVES", "")])
def test_tuning_variables_are_parsed_strictly(var, val, monkeypatch):
    monkeypatch.setenv(var, val)
    assert call_decode(shape()) == -3
    assert pa.variant_name(shape(), 128, 16) is None


def test_empty_batch_is_ok_without_launch():
    assert call_decode(shape(num_seqs=0), q=None, out=None) == 0


def test_reduce_rejects():
    r = pa.lib().paged_attn_reduce
    s = shape(partition_size=512, max_partitions=4)
    assert r(None, 128, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert r(ctypes.byref(shape()), 128, FAKE, FAKE, FAKE, FAKE, None, None) == -2   # unsplit
    assert r(ctypes.byref(s), 96, FAKE, FAKE, FAKE, FAKE, None, None) == -3
    assert r(ctypes.byref(s), 128, None, FAKE, FAKE, FAKE, None, None) == -1
    assert r(ctypes.byref(s), 128, FAKE, FAKE, FAKE, None, None, None) == -1
    assert r(ctypes.byref(shape(num_seqs=0, partition_size=512, max_partitions=4)), 128,
             None, None, None, None, None, None) == 0


def test_debug_entry_points_reject():
    lib = pa.lib()
    assert lib.paged_attn_stream_read(None, 1024, 4, FAKE, None) == -1
    assert lib.paged_attn_stream_read(FAKE, 1000, 4, FAKE, None) == -2
    assert lib.paged_attn_stream_read(FAKE, 1024, 0, FAKE, None) == -2
    assert lib.paged_attn_copy(FAKE, None, 16, None) == -1
    assert lib.paged_attn_copy(FAKE, FAKE, 15, None) == -2
    s = shape()
    w = lib.paged_attn_gather_witness
    assert w(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 96, 16, 0, 8, FAKE, FAKE, None) == -3
    assert w(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 128, 16, 0, 0, FAKE, FAKE, None) == -2
    assert w(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 128, 16, 0, 8, None, FAKE, None) == -1


# ---------------------------------------------------------------------------------------------
# host table check
# ---------------------------------------------------------------------------------------------
def test_check_tables():
    bt = np.array([[3, 1, 7, -1], [0, 2, 31, 5]], np.int32)
    L = np.array([40, 64], np.int32)
    s = shape(block_table_stride=4)
    assert pa.check_tables(s, 16, 0, bt, L) == 0                     # entry 3 of row 0 unread
    assert pa.check_tables(s, 16, 0, bt, np.array([49, 64], np.int32)) == -6   # reads -1
    bad = bt.copy()
    bad[1, 3] = 32
    assert pa.check_tables(s, 16, 0, bad, L) == -6                   # id == num_blocks
    assert pa.check_tables(s, 16, 0, bt, np.array([40, 65], np.int32)) == -6   # L > stride*bs
    assert pa.check_tables(s, 16, 0, bt, np.array([-1, 3], np.int32)) == -6
    # the window skips blocks before its start: a bad entry there is never read
    pre = bt.copy()
    pre[1, 0] = -5
    assert pa.check_tables(s, 16, 0, pre, L) == -6
    assert pa.check_tables(s, 16, 40, pre, L) == 0
    sp = shape(block_table_stride=4, partition_size=32, max_partitions=1)
    assert pa.check_tables(sp, 16, 0, bt, L) == -6                   # needs 2 partitions
    assert pa.check_tables(shape(block_table_stride=4, partition_size=32, max_partitions=2),
                           16, 0, bt, L) == 0


def test_suggest_partition_size():
    for B, hkv, L, bs in [(64, 8, 4096, 16), (4, 8, 131072, 64), (32, 8, 8192, 16),
                          (1, 4, 2048, 16), (128, 8, 32768, 16)]:
        P = pa.suggest_partition_size(B, hkv, L, bs, 256)
        assert P == 0 or (P % bs == 0 and P % 16 == 0 and 256 <= P <= 2048), (B, L, P)
    assert pa.suggest_partition_size(512, 8, 512, 16, 256) == 0
    assert pa.suggest_partition_size(0, 8, 512, 16, 256) == 0


# ---------------------------------------------------------------------------------------------
# the Python binding refuses what the library cannot take, before calling it
# ---------------------------------------------------------------------------------------------
def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(32, 2, 16, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 8, dtype=torch.int32)
    L = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.decode(q, k, k, bt, L, 0.1)


# ---------------------------------------------------------------------------------------------
# balanced schedule: host-side validation
# ---------------------------------------------------------------------------------------------
def call_balanced(s, *, head_dim=128, block_size=16, window=0, ws=FAKE, ws_bytes=1 << 30,
                  workers=64, out=FAKE):
    return pa.lib().paged_attn_decode_balanced(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE,
                                               0.1, head_dim, block_size, window, None, out,
                                               None, ws, ws_bytes, workers, None)


def test_balanced_workspace_size_formula():
    s = shape(num_seqs=5, num_q_heads=8, num_kv_heads=2)
    n = pa.balanced_workspace_size(s, 128, 100)
    # prefix int64[B+1] | lse f32[N][2][G] | o f32[N][2][G][D], each 256-byte aligned
    a = lambda x: (x + 255) // 256 * 256
    assert n == a(6 * 8) + a(100 * 2 * 4 * 4) + a(100 * 2 * 4 * 128 * 4)
    with pytest.raises(pa.PagedAttnError):
        pa.balanced_workspace_size(s, 96, 100)
    with pytest.raises(pa.PagedAttnError):
        pa.balanced_workspace_size(s, 128, -1)


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=96), -3), (dict(block_size=8), -3), (dict(window=-2), -2),
    (dict(workers=-1), -2), (dict(workers=(1 << 20) + 1), -2),
    (dict(ws=None), -1), (dict(out=None), -1),
    (dict(ws=ctypes.c_void_p(0x1004)), -2),          # misaligned
    (dict(ws_bytes=1024), -2),                        # too small for 64 workers
])
def test_balanced_rejects(kw, expect):
    assert call_balanced(shape(), **kw) == expect


def test_balanced_empty_batch_is_ok_without_launch():
    assert call_balanced(shape(num_seqs=0), ws=None, out=None) == 0


def call_noalloc(s, *, head_dim=128, block_size=16, window=0, workers=64, q=FAKE, out=FAKE,
                 scale=0.1):
    return pa.lib().paged_attn_decode_balanced_noalloc(ctypes.byref(s), q, FAKE, FAKE, FAKE,
                                                       FAKE, scale, head_dim, block_size, window,
                                                       None, out, None, workers, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=96), -3), (dict(block_size=8), -3), (dict(window=-2), -2),
    (dict(workers=-1), -2), (dict(workers=(1 << 20) + 1), -2), (dict(scale=float("nan")), -2),
    (dict(q=None), -1), (dict(out=None), -1),
    # partials beyond the 32 MiB device array: 2 * 4 * 128 * 4 bytes per worker at G = 4
    (dict(workers=(32 << 20) // 4096 + 1), -2),
])
def test_noalloc_rejects_before_touching_the_device(kw, expect):
    """Every refusal of the no-allocation entry point comes from host checks (this machine has
    no GPU): bad sizes, NULL pointers, and partials too large for its device array."""
    assert call_noalloc(shape(), **kw) == expect
    assert pa.balanced_workspace_size(shape(), 128, (32 << 20) // 4096 + 1) > 32 << 20


def test_noalloc_empty_batch_is_ok_without_launch():
    assert call_noalloc(shape(num_seqs=0), q=None, out=None) == 0


# ---------------------------------------------------------------------------------------------
# prepared decode (plans): creation-time checks, workspace sizes, run-time argument checks
# ---------------------------------------------------------------------------------------------
def plan_create(s, *, head_dim=128, block_size=16, window=0, schedule=0, workers=0, max_len=0,
                kv_dtype=0, q_len=1, layout=None):
    h = ctypes.c_void_p()
    lay = None if layout is None else ctypes.byref(pa.KvLayout(*layout))
    st = pa.lib().paged_attn_plan_create(ctypes.byref(s), head_dim, block_size, window, schedule,
                                         kv_dtype, lay, q_len, max_len, workers, ctypes.byref(h))
    return st, h


def test_query_block_plans():
    # one wave per (sequence, KV head, 32 / group tokens; 16 / group at D = 256), no workspace
    st, h = plan_create(shape(), schedule=4, q_len=70)
    assert st == 0
    assert pa.lib().paged_attn_plan_workspace_size(h) == 0
    # 70 tokens = 9 blocks of 8: workgroups of four waves sharing the tiles through LDS
    assert pa.lib().paged_attn_plan_name(h) == b"pa_qblock_mfmapv_d128_g4_q70_t8_w4"
    pa.lib().paged_attn_plan_destroy(h)
    # 5 tokens = 2 blocks of 4: one wave per block
    st, h = plan_create(shape(), schedule=4, q_len=5, head_dim=256, kv_dtype=1)
    assert st == 0
    assert pa.lib().paged_attn_plan_name(h) == b"pa_qblock_mfmapv_fp8_d256_g4_q5_t4_w1"
    pa.lib().paged_attn_plan_destroy(h)
    # 4 sequences x 2 KV heads = 8 units: every block of a unit on one XCD
    st, h = plan_create(shape(num_seqs=4), schedule=4, q_len=1)
    assert st == 0 and pa.lib().paged_attn_plan_name(h).endswith(b"_xcd")
    pa.lib().paged_attn_plan_destroy(h)
    assert plan_create(shape(partition_size=512, max_partitions=4), schedule=4, q_len=3)[0] == -2
    assert plan_create(shape(), schedule=4, q_len=0)[0] == -2
    assert plan_create(shape(), schedule=4, q_len=4097)[0] == -2
    assert plan_create(shape(), schedule=5, q_len=3)[0] == -2
    assert plan_create(shape(), schedule=4, q_len=3, head_dim=96)[0] == -3



def test_plan_flags_one_term_p():
    """PA_PLAN_P_ONE_BF16 reaches the 32-key workgroup form only (bf16 caches, head_dim <= 128,
    four or more blocks per (sequence, KV head)); other plans ignore it; unknown bits are
    rejected."""
    def create(flags, **kw):
        h = ctypes.c_void_p()
        st = pa.lib().paged_attn_plan_create_flags(
            ctypes.byref(shape(**kw.pop("shape_kw", {}))), kw.get("head_dim", 128), 16, 0,
            kw.get("schedule", 4), kw.get("kv_dtype", 0), None, kw.get("q_len", 70), 0, 100,
            flags, ctypes.byref(h))
        name = pa.lib().paged_attn_plan_name(h) if st == 0 else None
        if st == 0:
            pa.lib().paged_attn_plan_destroy(h)
        return st, name

    assert create(1) == (0, b"pa_qblock_mfmapv_d128_g4_q70_t8_w4_p1")
    assert create(0) == (0, b"pa_qblock_mfmapv_d128_g4_q70_t8_w4")
    assert create(1, head_dim=64) == (0, b"pa_qblock_mfmapv_d64_g4_q70_t8_w4_p1")
    # FP8 caches, head_dim 256 and one wave per block keep both terms
    assert create(1, kv_dtype=1)[1] == b"pa_qblock_mfmapv_fp8_d128_g4_q70_t8_w4"
    assert not create(1, head_dim=256)[1].endswith(b"_p1")
    assert create(1, q_len=5)[1] == b"pa_qblock_mfmapv_d128_g4_q5_t8_w1"
    # other schedules ignore the bit
    st, name = create(1, schedule=2, q_len=1)
    assert st == 0 and b"_p1" not in name and b"workers100" in name
    # unknown bits
    assert create(2)[0] == -3
    assert create(1 << 30)[0] == -3
    # paged_attn_plan_create is the flags call with no bits
    st, h = plan_create(shape(), schedule=4, q_len=70)
    assert st == 0 and pa.lib().paged_attn_plan_name(h) == b"pa_qblock_mfmapv_d128_g4_q70_t8_w4"
    pa.lib().paged_attn_plan_destroy(h)


def test_query_block_key_splits():
    """Small batches cut each block's key range into key splits (about 2048 waves in all, at
    least 8 tiles a split, at most 64 splits) and take a workspace for the partials."""
    a = lambda x: (x + 255) // 256 * 256

    def check(s, q_len, max_len, window=0, head_dim=128):
        st, h = plan_create(s, schedule=4, q_len=q_len, max_len=max_len, window=window,
                            head_dim=head_dim)
        assert st == 0
        name = pa.lib().paged_attn_plan_name(h).decode()
        ws = pa.lib().paged_attn_plan_workspace_size(h)
        pa.lib().paged_attn_plan_destroy(h)
        return name, ws

    # B2, 2 KV heads, group 4, 70 tokens: 3 workgroups of four waves per (sequence, KV head),
    # 48 waves; 8192 keys = 513 tiles (one straddled) -> 43 splits of 12 tiles
    name, ws = check(shape(), 70, 8192)
    assert name == "pa_qblock_mfmapv_d128_g4_q70_t8_w4_s43"
    slots = 2 * 70 * 8 * 43
    assert ws == a(slots * 128 * 4) + a(slots * 4)
    # one token per block at the most: 2 blocks of 4 tokens, 8 waves -> capped at 64 splits
    name, ws = check(shape(), 5, 131072, head_dim=256)
    assert name.endswith("_w1_s64")
    assert ws == a(2 * 5 * 8 * 64 * 256 * 4) + a(2 * 5 * 8 * 64 * 4)
    # unknown lengths, short lengths, a short window, a large batch: no split, no workspace
    for s_, q, L, w in ((shape(), 70, 0, 0), (shape(), 2, 64, 0), (shape(), 70, 8192, 100),
                        (shape(num_seqs=512, block_table_stride=8), 70, 8192, 0)):
        name, ws = check(s_, q, L, w)
        assert "_s" not in name.replace("_xcd", "") and ws == 0, (name, ws)


# (B, Hq, Hkv, D, bs, window, q_len, max_seq_len) -> (schedule, partition_size) on 256 CUs
SUGGESTIONS = [
    ((2, 4, 2, 128, 16, 0, 1, 100), ("unsplit", 0)),          # tiny: one short range each
    ((128, 32, 8, 128, 16, 0, 1, 256), ("unsplit", 0)),
    ((32, 32, 8, 128, 16, 0, 1, 1024), ("unsplit", 0)),       # 256 units cover the CUs
    ((1, 32, 8, 128, 16, 0, 1, 2048), ("partitioned", 256)),  # little work: latency case
    ((4, 32, 4, 128, 16, 0, 1, 16384), ("partitioned", 256)),  # 16 units x 16384 = 1024 / CU
    ((4, 32, 4, 128, 64, 0, 1, 16384), ("partitioned", 256)),
    ((1, 32, 8, 128, 256, 0, 1, 2048), ("partitioned", 256)),
    ((4, 32, 8, 128, 16, 0, 1, 16384), ("balanced", 0)),      # 32 units x 16384: past that
    ((64, 32, 8, 128, 16, 0, 1, 4096), ("balanced", 0)),      # the Llama-8B-shaped step
    ((128, 32, 8, 128, 16, 4096, 1, 32768), ("balanced", 0)),  # window 4096
    ((128, 32, 8, 128, 16, 200, 1, 32768), ("unsplit", 0)),   # the window bounds the keys
    ((64, 32, 8, 128, 16, 0, 1, 0), ("balanced", 0)),         # no bound given
    ((1, 32, 8, 128, 16, 0, 4, 8192), ("balanced", 0)),       # 16 pairs: one balanced pass
    ((1, 32, 8, 128, 16, 0, 8, 8192), ("balanced", 0)),       # 32 pairs, small batch
    ((16, 32, 8, 128, 16, 0, 8, 2048), ("query_blocks", 0)),  # 32 pairs, 128 units
    ((1, 32, 8, 128, 16, 0, 16, 8192), ("query_blocks", 0)),
    ((1, 32, 8, 256, 16, 0, 4, 8192), ("balanced", 0)),       # 16 pairs fill a D=256 block,
    ((16, 32, 8, 256, 16, 0, 4, 8192), ("query_blocks", 0)),  # a small batch stays balanced
    ((1, 32, 8, 256, 16, 0, 2, 8192), ("balanced", 0)),
    ((1, 16, 2, 128, 16, 0, 8, 8192), ("query_blocks", 0)),   # group 8: 64 pairs
]


@pytest.mark.parametrize("args,expected", SUGGESTIONS)
def test_suggest_schedule(args, expected):
    B, Hq, Hkv, D, bs, W, Q, L = args
    assert pa.suggest_schedule(B, Hq, Hkv, D, bs, window=W, q_len=Q, max_seq_len=L,
                               num_cus=256) == expected


def test_suggest_schedule_rejects_bad_arguments():
    P = ctypes.c_int32(7)
    f = pa.lib().paged_attn_suggest_schedule
    assert f(1, 32, 8, 128, 16, 0, 1, 100, 256, None) == -1              # PA_ERR_NULL
    assert f(1, 30, 8, 128, 16, 0, 1, 100, 256, ctypes.byref(P)) == -2   # Hq % Hkv
    assert P.value == 0
    assert f(1, 32, 8, 128, 16, -1, 1, 100, 256, ctypes.byref(P)) == -2  # window
    assert f(1, 32, 8, 128, 16, 0, 0, 100, 256, ctypes.byref(P)) == -2   # q_len
    assert f(1, 32, 8, 96, 16, 0, 1, 100, 256, ctypes.byref(P)) == -3    # head_dim
    assert f(1, 32, 8, 128, 24, 0, 1, 100, 256, ctypes.byref(P)) == -3   # block size
    # groups no kernel takes (plan creation rejects them too): nothing is suggested
    for hq, hkv, q in ((64, 2, 2), (128, 2, 2), (48, 8, 1), (16, 1, 1)):
        assert f(1, hq, hkv, 128, 16, 0, q, 8192, 256, ctypes.byref(P)) == -3, (hq, hkv)
    with pytest.raises(ValueError):
        pa.Plan(1, 32, 8, 10, 8, 128, 16, schedule="fastest")

def test_plan_create_and_workspace_sizes():
    a = lambda x: (x + 255) // 256 * 256
    st, h = plan_create(shape())
    assert st == 0 and h.value
    assert pa.lib().paged_attn_plan_workspace_size(h) == 0
    assert pa.lib().paged_attn_plan_name(h).decode().startswith("pa_decode_")
    pa.lib().paged_attn_plan_destroy(h)
    s = shape(partition_size=512, max_partitions=4)
    st, h = plan_create(s, schedule=1)
    assert st == 0
    rows = 2 * 8 * 4
    assert pa.lib().paged_attn_plan_workspace_size(h) == a(rows * 128 * 4) + a(rows * 4)
    assert b"pa_reduce" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    st, h = plan_create(s, schedule=3)
    assert st == 0
    assert pa.lib().paged_attn_plan_workspace_size(h) == \
        a(rows * 128 * 4) + a(rows * 4) + a(2 * 2 * 4)
    assert b"last partition" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    # one bf16 token at head_dim 128: one KV head per unit, the eager call's workspace
    st, h = plan_create(shape(), schedule=2, workers=100)
    assert st == 0
    assert pa.lib().paged_attn_plan_workspace_size(h) == pa.balanced_workspace_size(shape(), 128,
                                                                                     100)
    assert b"mfmapv_d128_g4_workers100" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    # at head_dim 64 (bf16 or FP8), 2 KV heads of 4 query heads form one KV-head pair per
    # sequence: 8 columns, the workspace of a shape with one KV head of 8
    # query heads
    for hd, kvd, tag in ((64, 0, b"mfmapv_headpairs_d64_g4_workers100"),
                         (64, 1, b"mfmapv_fp8_headpairs_d64_g4_workers100")):
        st, h = plan_create(shape(), schedule=2, workers=100, head_dim=hd, kv_dtype=kvd)
        assert st == 0 and tag in pa.lib().paged_attn_plan_name(h)
        assert pa.lib().paged_attn_plan_workspace_size(h) == pa.balanced_workspace_size(
            shape(num_kv_heads=1), hd, 100)
        pa.lib().paged_attn_plan_destroy(h)
    # no pairs for an odd number of KV heads (the workspace of the eager call)
    st, h = plan_create(shape(num_q_heads=12, num_kv_heads=3), schedule=2, workers=100,
                        head_dim=64)
    assert st == 0 and b"headpairs" not in pa.lib().paged_attn_plan_name(h)
    assert pa.lib().paged_attn_plan_workspace_size(h) == pa.balanced_workspace_size(
        shape(num_q_heads=12, num_kv_heads=3), 64, 100)
    pa.lib().paged_attn_plan_destroy(h)
    # a length bound caps the workers: 2 seqs x 2 KV heads x (7 + 1) tiles / 4 = 8, and 4 with
    # KV-head pairs (one pair per sequence)
    st, h = plan_create(shape(), schedule=2, workers=100, max_len=100)
    assert st == 0 and b"workers8 " in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    st, h = plan_create(shape(), schedule=2, workers=100, max_len=100, head_dim=64)
    assert st == 0 and b"workers4 " in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    # an FP8 cache: the FP8 path under every schedule, the same workspace as bf16
    for sched, sh in ((0, shape()), (1, s), (3, s)):
        st, h = plan_create(sh, schedule=sched, kv_dtype=1)
        st16, h16 = plan_create(sh, schedule=sched)
        assert st == 0 and st16 == 0
        assert b"mfmapv_fp8" in pa.lib().paged_attn_plan_name(h)
        assert pa.lib().paged_attn_plan_workspace_size(h) == \
            pa.lib().paged_attn_plan_workspace_size(h16)
        pa.lib().paged_attn_plan_destroy(h)
        pa.lib().paged_attn_plan_destroy(h16)
    st, h = plan_create(shape(), schedule=2, workers=100, kv_dtype=1)
    assert st == 0 and pa.lib().paged_attn_plan_name(h).startswith(b"pa_balanced_mfmapv_fp8_")
    pa.lib().paged_attn_plan_destroy(h)
    # several query tokens: (token, head) columns rounded up to a power of two, the workspace
    # sized for them; 3 tokens x 4 heads -> 16 columns
    st, h = plan_create(shape(), schedule=2, workers=100, q_len=3)
    assert st == 0 and b"_g4_q3_c16_workers100" in pa.lib().paged_attn_plan_name(h)
    a = lambda x: (x + 255) // 256 * 256
    ws = a(3 * 8) + a(100 * 2 * 16 * 4) + a(100 * 2 * 16 * 128 * 4)
    assert pa.lib().paged_attn_plan_workspace_size(h) == ws
    pa.lib().paged_attn_plan_destroy(h)
    # 17 to 32 columns: one pass of the two-half kernels at D <= 128; more: passes of
    # 32 / group tokens (here 8 + 1), or of 16 / group at D = 256 (4 + 4 + 1)
    st, h = plan_create(shape(), schedule=2, workers=100, q_len=8)
    assert st == 0 and b"_g4_q8_c32_workers100" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    st, h = plan_create(shape(), schedule=2, workers=100, q_len=9)
    assert st == 0 and b"_g4_q9_c32_passes2_workers100" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    st, h = plan_create(shape(), schedule=2, workers=100, q_len=9, head_dim=256)
    assert st == 0 and b"_g4_q9_c16_passes3_workers100" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    st, h = plan_create(shape(), schedule=2, workers=100, q_len=2, kv_dtype=1)
    assert st == 0 and b"mfmapv_fp8_d128_g4_q2_c8" in pa.lib().paged_attn_plan_name(h)
    pa.lib().paged_attn_plan_destroy(h)
    # KV layouts: token-major, K/V interleaved per block, padded rows; FP8 token-major
    for sched, lay, kv in ((0, (16 * 2 * 128, 128, 2 * 128), 0), (2, (2 * 2 * 16 * 128, 16 * 128, 128), 0),
                           (1, (2 * 16 * 136, 16 * 136, 136), 0), (2, (16 * 2 * 128, 128, 256), 1)):
        sh = shape(partition_size=512, max_partitions=4) if sched == 1 else shape()
        st, h = plan_create(sh, schedule=sched, workers=64, layout=lay, kv_dtype=kv)
        assert st == 0, (sched, lay, kv)
        pa.lib().paged_attn_plan_destroy(h)
    pa.lib().paged_attn_plan_destroy(None)


@pytest.mark.parametrize("kw,expect", [
    (dict(schedule=1), -2),                      # partitioned without a partition size
    (dict(schedule=3), -2), (dict(schedule=5), -2), (dict(schedule=-1), -2),
    (dict(head_dim=96), -3), (dict(block_size=8), -3), (dict(window=-1), -2),
    (dict(schedule=2, workers=-1), -2), (dict(schedule=2, workers=(1 << 20) + 1), -2),
    (dict(max_len=-1), -2), (dict(kv_dtype=2), -3), (dict(kv_dtype=-1), -3),
    (dict(q_len=0), -2), (dict(q_len=-3), -2),
    (dict(q_len=2), -3),                         # several query tokens: balanced or query
                                                 # blocks only
    (dict(q_len=4097, schedule=2, workers=64), -2),  # above 4096 query tokens
    (dict(q_len=2, schedule=2, workers=64, window=0x7FFFFFFF), -2),
    # layouts (elements; head_dim 128, block 16, 2 KV heads)
    (dict(layout=(4096, 2048, 120)), -2),          # token stride below head_dim
    (dict(layout=(0, 2048, 128)), -2), (dict(layout=(4096, -1, 128)), -2),
    (dict(layout=(4096, 2048, 132)), -2),          # 264-byte rows: not 16-byte aligned
    (dict(layout=(4100, 2048, 128)), -2),          # block stride not 16-byte aligned
    (dict(layout=(4096, 2048, 136), kv_dtype=1), -2),   # FP8: 136-byte rows
    (dict(layout=(4096, 2048, 1 << 26)), -2),      # row stride above 2^26 bytes
])
def test_plan_create_rejects(kw, expect):
    st, h = plan_create(shape(), **kw)
    assert st == expect and not h.value


def test_plan_unsplit_rejects_a_partitioned_shape_and_null_out_pointer():
    st, h = plan_create(shape(partition_size=512, max_partitions=4), schedule=0)
    assert st == -2
    s = shape()
    assert pa.lib().paged_attn_plan_create(ctypes.byref(s), 128, 16, 0, 0, 0, None, 1, 0, 0,
                                           None) == -1


def test_plan_run_argument_checks_without_launch():
    lib = pa.lib()
    st, h = plan_create(shape(), schedule=2, workers=64)
    assert st == 0
    # q k v table lens scale k_scale v_scale sinks out lse workspace stream
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1.0, 1.0, None, FAKE, None, FAKE, None]
    assert lib.paged_attn_plan_run(None, *args) == -1
    for i in (5, 6, 7):
        for v in (float("inf"), float("nan")):
            bad = list(args); bad[i] = v
            assert lib.paged_attn_plan_run(h, *bad) == -2, (i, v)
    for i in (6, 7):                          # a bf16 plan takes no KV scales
        bad = list(args); bad[i] = 0.5
        assert lib.paged_attn_plan_run(h, *bad) == -2, i
    for i in (0, 1, 2, 3, 4, 9):
        bad = list(args); bad[i] = None
        assert lib.paged_attn_plan_run(h, *bad) == -1, i
    bad = list(args); bad[11] = None          # balanced plans need a workspace
    assert lib.paged_attn_plan_run(h, *bad) == -1
    bad = list(args); bad[11] = ctypes.c_void_p(0x1010)   # not 256-byte aligned
    assert lib.paged_attn_plan_run(h, *bad) == -2
    lib.paged_attn_plan_destroy(h)
    st, h = plan_create(shape(num_seqs=0), schedule=2, workers=64)
    assert st == 0 and lib.paged_attn_plan_run(h, *([None] * 5 + [0.1, 1.0, 1.0] + [None] * 5)) == 0
    lib.paged_attn_plan_destroy(h)
    # an FP8 plan takes any finite scales; an empty batch returns before any launch
    st, h = plan_create(shape(num_seqs=0), schedule=0, kv_dtype=1)
    assert st == 0
    assert lib.paged_attn_plan_run(h, *([None] * 5 + [0.1, 0.03, -2.0] + [None] * 5)) == 0
    bad = [None] * 5 + [0.1, float("nan"), 1.0] + [None] * 5
    assert lib.paged_attn_plan_run(h, *bad) == -2
    lib.paged_attn_plan_destroy(h)


def test_plan_binding_refuses_host_tensors():
    plan = pa.Plan(2, 8, 2, 32, 8, 128, 16, schedule="unsplit")
    assert plan.workspace_size == 0 and plan.workspace("cpu") is None
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        plan.run(x, x, x, x, x, 0.1, out=x)
    with pytest.raises(ValueError):
        pa.Plan(2, 8, 2, 32, 8, 128, 16, schedule="partitioned")
    with pytest.raises(ValueError):
        pa.Plan(2, 8, 2, 32, 8, 128, 16, schedule="fast")
    with pytest.raises(ValueError):
        pa.Plan(2, 8, 2, 32, 8, 128, 16, schedule="unsplit", kv_dtype="fp8")

"""The no-allocation entry point (paged_attn_decode_balanced_noalloc) on the GPU: its results
equal those of the entry point it stands in for, paged_attn_decode_balanced +
paged_attn_reduce_balanced with a caller workspace (the same kernels and worker count, so bit
for bit), and the fp64 oracle to the contract and the regression gates; two calls in a row, the
second on a smaller batch, so that what the first leaves in the library's array cannot leak into
the second; and a shape whose partials do not fit is refused before anything is launched."""
import numpy as np
import pytest
import torch

import paged_kv_attention_attn_amd as pa
from workloads import make_config, make_workload

from gpu_helpers import compare, log, oracle_full, to_dev

pytestmark = pytest.mark.gpu


def _existing(wl, t, workers):
    B, Hq, D = wl.q.shape
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    pa.decode_balanced(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                       window=wl.window, sinks=t["sinks"], out=out, lse=lse,
                       num_workers=workers)
    torch.cuda.synchronize()
    return out, lse


def _noalloc(wl, t, workers):
    B, Hq, D = wl.q.shape
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    pa.decode_balanced_noalloc(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                               out=out, lse=lse, window=wl.window, sinks=t["sinks"],
                               num_workers=workers)
    torch.cuda.synchronize()
    return out, lse


def _check(wl, workers, tag):
    t = to_dev(wl)
    got = _noalloc(wl, t, workers)
    ref = _existing(wl, t, workers)
    log(f"[noalloc] {tag}: B={wl.num_seqs} workers={workers}")
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), tag
    compare(got[0].cpu().numpy().astype(np.float64), got[1].cpu().numpy().astype(np.float64),
            *oracle_full(wl), f"noalloc {tag}")


def test_noalloc_equals_the_workspace_entry_point_on_two_calls_in_a_row():
    # first the mixed batch (128 sequences, window and sinks), then a smaller one
    _check(make_config(5, poison=True), 0, "mixed batch B=128")
    small = make_workload(name="noalloc small", seq_lens=[1000, 3, 0, 4097, 17], num_q_heads=8,
                          num_kv_heads=2, head_dim=128, block_size=16, seed=[5, 1], window=0,
                          with_sinks=True, poison=True)
    _check(small, 37, "small batch B=5")


def test_noalloc_other_head_sizes_and_the_default_workload():
    _check(make_config(2, poison=True), 0, "Llama-8B step")
    for D, g in ((64, 8), (256, 4)):
        wl = make_workload(name=f"noalloc D{D}", seq_lens=[700, 1, 2049, 16, 0, 333],
                           num_q_heads=2 * g, num_kv_heads=2, head_dim=D, block_size=32,
                           seed=[D, g, 3], window=500, with_sinks=False, poison=True)
        _check(wl, 0, f"D={D} g={g}")


def test_noalloc_refuses_partials_that_do_not_fit():
    wl = make_workload(name="noalloc big", seq_lens=[64, 64], num_q_heads=16, num_kv_heads=2,
                       head_dim=256, block_size=16, seed=[9], poison=True)
    t = to_dev(wl)
    shape = pa.make_shape(2, 16, 2, wl.num_blocks, wl.stride)
    workers = 1 << 14      # 2 * 8 * 256 * 4 = 16 KiB of partials per worker: 256 MiB
    assert pa.balanced_workspace_size(shape, 256, workers) > 32 << 20
    out = torch.zeros((2, 16, 256), device="cuda")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.decode_balanced_noalloc(t["q"], t["k"], t["v"], t["bt"], t["L"], float(wl.scale),
                                   out=out, num_workers=workers)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert not out.any()   # nothing was launched

"""The measurement probes of the debug ABI on the GPU: the gather-read probe reads exactly the
chunks it is given (its checksums XOR to the XOR of those chunks' words, computed on the host)
and skips ids outside the buffer."""
import numpy as np
import pytest
import torch

from paged_kv_attention_attn_amd import debug

from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [2048, 4096, 8192])
@pytest.mark.parametrize("wg", [1, 7, 64])
def test_gather_read_reads_the_listed_chunks(chunk, wg):
    rng = np.random.default_rng(chunk + wg)
    n = 96
    host = rng.integers(0, 2 ** 32, size=n * chunk // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    ids = rng.permutation(n).astype(np.int32)
    ids = np.concatenate([ids, [n, -1, n + 5]]).astype(np.int32)   # outside: skipped
    rng.shuffle(ids)
    sink = torch.zeros(wg, dtype=torch.int32, device="cuda")
    debug.gather_read(buf, chunk, torch.from_numpy(ids).cuda(), wg, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    log(f"[probe] gather_read chunk={chunk} wg={wg}: {got:#x} vs {want:#x}")
    assert got == want
    # a list with one chunk twice and one chunk once: the twice-read chunk cancels
    ids2 = torch.tensor([3, 3, 10], dtype=torch.int32, device="cuda")
    debug.gather_read(buf, chunk, ids2, wg, sink)
    torch.cuda.synchronize()
    words = host.reshape(n, chunk // 4)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == \
        np.bitwise_xor.reduce(words[10])

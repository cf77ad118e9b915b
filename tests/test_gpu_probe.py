"""GPU: the read probe (pa_probe_read) reads every byte it is asked to, once.

Each thread XORs the 16-byte vectors it reads and stores one word, so the XOR
of all stored words equals the XOR of every 32-bit word read: the buffer's own
XOR when every vector is read exactly once.  Integer work, compared exactly.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_117_amd as pa

pytestmark = pytest.mark.gpu


def _xor_all(a):
    return int(np.bitwise_xor.reduce(np.asarray(a, dtype=np.uint32).ravel()))


def _buffer(nchunks, seed):
    rng = np.random.default_rng(seed)
    host = rng.integers(0, 2**32, size=nchunks * 1024, dtype=np.uint32)
    return host, torch.from_numpy(host.view(np.int32)).cuda()


@pytest.mark.parametrize("nchunks,wg", [(1, 1), (13, 1), (64, 3), (257, 8)])
def test_sequential_reads_every_word_once(nchunks, wg):
    print(f"case sequential nchunks={nchunks} wg={wg}", flush=True)
    host, buf = _buffer(nchunks, seed=nchunks)
    sink = torch.zeros(wg * 256, dtype=torch.int32, device="cuda")
    pa.probe_read(buf, sink, wg)
    torch.cuda.synchronize()
    assert _xor_all(sink.cpu().numpy().view(np.uint32)) == _xor_all(host)


@pytest.mark.parametrize("nchunks,wg", [(13, 1), (64, 3), (257, 8)])
def test_gather_reads_each_listed_chunk_and_skips_invalid_entries(nchunks, wg):
    print(f"case gather nchunks={nchunks} wg={wg}", flush=True)
    host, buf = _buffer(nchunks, seed=100 + nchunks)
    rng = np.random.default_rng(nchunks)
    perm = rng.permutation(nchunks).astype(np.int32)
    # a permutation of every chunk plus out-of-range entries, which are skipped
    order = np.concatenate([perm[: nchunks // 2], [-1, nchunks, 2**31 - 1], perm[nchunks // 2:]]).astype(np.int32)
    sink = torch.zeros(wg * 256, dtype=torch.int32, device="cuda")
    pa.probe_read(buf, sink, wg, torch.from_numpy(order).cuda())
    torch.cuda.synchronize()
    assert _xor_all(sink.cpu().numpy().view(np.uint32)) == _xor_all(host)
    # a subset: only the listed chunks count
    sub = perm[: max(1, nchunks // 3)]
    pa.probe_read(buf, sink, wg, torch.from_numpy(sub).cuda())
    torch.cuda.synchronize()
    want = _xor_all(host.reshape(nchunks, 1024)[sub])
    assert _xor_all(sink.cpu().numpy().view(np.uint32)) == want

"""The read probe (a measurement aid of bench.py --read-bw) reads exactly the
bytes it claims: its per-thread xor folds match a NumPy replay of the access
pattern, for the streaming form (with a ragged tail) and the block form."""

import numpy as np
import pytest
import torch

from causal_streaming_decoding_amd import wedlm as W_

pytestmark = pytest.mark.gpu


def _src(nbytes, seed):
    rng = np.random.default_rng(seed)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    return host, torch.from_numpy(host.view(np.int32).copy()).cuda()


def test_stream_probe_reads_every_vector_once():
    nbytes = 16 * (256 * 3 * 4 + 37)      # four vectors per thread and a ragged tail
    host, src = _src(nbytes, 1)
    grid = 3
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    W_.wedlm_read_probe(src, nbytes, None, 0, sink, grid)
    torch.cuda.synchronize()
    vec = host.reshape(-1, 4)
    stride = grid * 256
    expect = np.zeros(stride, np.uint32)
    for t in range(stride):
        acc = np.bitwise_xor.reduce(vec[t::stride], axis=0) if t < len(vec) else np.zeros(4, np.uint32)
        expect[t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), expect)


def test_block_probe_follows_the_order():
    n_src = 40
    nbytes = n_src * 4096
    host, src = _src(nbytes, 2)
    order = np.array([5, 0, 39, 7, 7, 12, 33, 2, 19], np.int32)
    grid = 1                               # 4 waves, so waves 0 and 1 take two blocks
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    W_.wedlm_read_probe(src, nbytes, torch.from_numpy(order).cuda(), len(order), sink, grid)
    torch.cuda.synchronize()
    vec = host.reshape(n_src, 256, 4)
    expect = np.zeros(256, np.uint32)
    for w in range(4):
        for lane in range(64):
            acc = np.zeros(4, np.uint32)
            for j in range(w, len(order), 4):
                for u in range(4):
                    acc ^= vec[order[j], lane + 64 * u]
            expect[w * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3]
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), expect)

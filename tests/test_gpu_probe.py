"""The streaming-read probe (cbd_read_probe): every thread's XOR fold of the
16-byte words it reads (words tid, tid + G, ... of G = blocks x 1024
threads) equals the same fold taken on the host, so every word of the
buffer was read exactly once by the thread the layout assigns it to."""
import numpy as np
import pytest
import torch

from continuous_batching_decode_forward_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 4), ((1 << 20) + 48, 3)])
def test_read_probe_folds_every_word(nbytes, blocks):
    g = np.random.default_rng(nbytes)
    host = g.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    G = blocks * 1024
    out = torch.full((G,), -1, dtype=torch.int32, device="cuda")
    B.cbd_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    words = host.view(np.uint32).reshape(-1, 4)
    fold = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    want = np.zeros(G, np.uint32)
    n16 = len(fold)
    for t0 in range(0, n16, G):
        part = fold[t0:t0 + G]
        want[:len(part)] ^= part
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)

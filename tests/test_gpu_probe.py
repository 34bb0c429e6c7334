"""The stream-read probe the benchmark's measured read ceiling comes from:
it must read every word of the buffer once (its XOR fold equals the host's)."""
import numpy as np
import pytest
import torch

import free_sparse_swiglu_stage1_amd as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 1 << 10, (1 << 20) + 4, 3 * (1 << 22) + 12])
def test_read_probe_reads_every_word(n_words):
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 32, size=n_words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.read_probe(buf, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(expect)

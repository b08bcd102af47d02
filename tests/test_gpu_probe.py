"""The streaming-read probe (a measurement utility) reads every word of its buffer: the XOR of
its per-workgroup sink words equals the XOR of the buffer's words, for a buffer with a ragged
tail (not a multiple of the grid's stride)."""

import numpy as np
import pytest
import torch


@pytest.mark.gpu
def test_read_probe_reads_every_word(gpu):
    import compressed_sparse_long_c4a_amd as csa
    print("case read_probe 3,000,004 words", flush=True)
    g = torch.Generator().manual_seed(5)
    host = torch.randint(-2**31, 2**31 - 1, (3_000_004,), generator=g, dtype=torch.int64).to(torch.int32)
    sink = csa.read_probe(host.cuda())
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want

"""GPU check of the HBM read-stream reference.  A thread writes the sink
only when the XOR of the words it read equals a fixed constant, so a buffer
of zeros with that constant in one 16-byte word shows that the word was
read, at the start, the end (the ragged tail after the unrolled grid-stride
steps) and in between."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_compress_amd as kvc
from helpers import say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 22) + 16 * 7, (3 << 26) + 16 * 333])
def test_read_stream_reads_every_word(nbytes):
    say(f"[read_stream] bytes={nbytes}")
    n16 = nbytes // 16
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    kvc.kv_read_stream(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0
    g = np.random.default_rng(nbytes)
    for word in sorted({0, n16 - 1, int(g.integers(0, n16))}):
        buf.zero_()
        buf[4 * word] = np.int32(np.uint32(MAGIC).view(np.int32))
        sink.zero_()
        kvc.kv_read_stream(buf, nbytes, sink)
        torch.cuda.synchronize()
        assert int(sink[0]) & 0xFFFFFFFF == MAGIC, word

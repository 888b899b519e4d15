"""The read-ceiling probe (tp_stream_read) reads every byte of its buffer
exactly once: the XOR of its sink equals the XOR, over the buffer's 16-byte
chunks, of each chunk's first and last 32-bit words (computed on the host)."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from tests.gpu_util import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kib", [1, 3, 4099, 12345, 65536])
def test_stream_read_reads_every_chunk_once(kib):
    T = torch()
    rng = np.random.default_rng(kib)
    host = rng.integers(0, 2**32, size=kib * 256, dtype=np.uint32)
    buf = T.from_numpy(host.view(np.int32)).cuda()
    sink = tp.stream_read(buf)
    T.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    chunks = host.reshape(-1, 4)
    want = np.bitwise_xor.reduce(chunks[:, 0] ^ chunks[:, 3])
    assert got == want


def test_stream_read_rejects_ragged_size():
    T = torch()
    buf = T.zeros(1000, dtype=T.uint8, device="cuda")
    with pytest.raises(tp.TPError, match="MISALIGNED"):
        tp.stream_read(buf)

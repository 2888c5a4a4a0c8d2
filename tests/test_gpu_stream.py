"""moe_stream_read, the streaming-read measurement aid: it must read every
byte of the buffer exactly once.  The XOR of all sink words equals the XOR
of all 32-bit words of the buffer (every word goes into exactly one
thread's XOR), for sizes with a ragged tail, below one load per thread and
above one unrolled sweep of the grid."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 7, 2048 * 256 * 16 * 8 * 2 + 16 * 123])
def test_stream_read_reads_every_word_once(dev, m, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.full((m.MOE_STREAM_SINK_WORDS,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    m.moe_stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_misuse(dev, m):
    src = torch.zeros(64, dtype=torch.uint8, device=dev)
    sink = torch.empty(m.MOE_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    assert m.lib.moe_stream_read(src.data_ptr(), 20, sink.data_ptr(), None) == m.MOE_EINVAL
    assert m.lib.moe_stream_read(src.data_ptr() + 4, 16, sink.data_ptr(), None) == m.MOE_EINVAL
    assert m.lib.moe_stream_read(None, 16, sink.data_ptr(), None) == m.MOE_EINVAL
    assert m.lib.moe_stream_read(src.data_ptr(), 0, None, None) == m.MOE_OK

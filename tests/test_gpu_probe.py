"""The streaming-read probe reads every byte once: the XOR of its per-work-group
words equals the XOR of the buffer's 32-bit words (numpy on the host)."""
import numpy as np
import pytest

import sparse_long_context_ffd_amd as ffd
from sparse_long_context_ffd_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 * 16, (1 << 20) + 48, 3 * (1 << 22) + 16 * 777])
def test_stream_read_checksum(nbytes):
    import torch
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=max(nbytes, 16), dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    sink = torch.full((_lib.STREAM_READ_SINK_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    L = ffd.lib()
    rc = L.ffd_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), None)
    assert rc == 0, ffd.strerror(rc)
    torch.cuda.synchronize()
    words = sink.cpu().numpy().view(np.uint32)
    expect = np.bitwise_xor.reduce(host[:nbytes].view(np.uint32)) if nbytes else np.uint32(0)
    assert np.bitwise_xor.reduce(words) == expect
    if nbytes == 0:
        assert not words.any()  # every work-group writes its (empty) XOR


def test_stream_read_binding():
    import torch
    src = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    sink = torch.empty(_lib.STREAM_READ_SINK_BYTES, dtype=torch.uint8, device="cuda")
    ffd.stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(np.arange(1 << 16, dtype=np.uint32))
    with pytest.raises(ValueError):
        ffd.stream_read(src, sink[:100])

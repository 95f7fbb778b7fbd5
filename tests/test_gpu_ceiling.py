"""The streaming-read reference kernel reads every word of its buffer once:
the XOR of its sink words equals the XOR of the buffer's 32-bit words."""
import ctypes

import numpy as np
import pytest
import torch

from test_abi import ceiling_lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 4096, 16 * 256 * 1024 * 3 + 208, 64 << 20])
def test_read_ceiling_reads_every_word_once(nbytes):
    lib = ceiling_lib()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    words = int(lib.qbd_read_ceiling_sink_words())
    sink = torch.full((words,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print(f"read_ceiling nbytes={nbytes}", flush=True)
    assert lib.qbd_read_ceiling(buf.data_ptr(), nbytes, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    assert torch.equal(buf.cpu(), torch.from_numpy(host.view(np.int32)))  # read-only

"""Reference kernels of the measurement library: the streaming read reads
every word of its buffer once (the XOR of its sink words equals the XOR of
the buffer's 32-bit words), and every grid-wide handoff form hands the whole
vector over with no wait giving up."""
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


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_grid_handoff_hands_over_every_value(mode):
    lib = ceiling_lib()
    words = int(lib.qbd_grid_handoff_work_words())
    work = torch.full((words + 64,), -1, dtype=torch.int32, device="cuda")
    base = work.data_ptr()
    off = (-base) % 256 // 4  # 256-byte aligned start inside the buffer
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for phases in (0, 1, 37):
        print(f"grid_handoff mode={mode} phases={phases}", flush=True)
        assert lib.qbd_grid_handoff(mode, phases, base + 4 * off, stream) == 0
        torch.cuda.synchronize()
        w = work[off:off + words].cpu().numpy().view(np.uint32)
        assert w[words - 64] == 0, "a wait gave up"
        assert w[words - 63] == 0, "vector values read back wrong"
        if phases:
            data = w[1024:3072].view(np.float32)
            last = (phases - 1) & 1
            assert np.array_equal(data[last * 1024:(last + 1) * 1024], np.arange(1024) * 7.0 + phases - 1)


def test_empty_launch():
    lib = ceiling_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.qbd_empty_launch(stream) == 0
    torch.cuda.synchronize()

"""The allocation-free entry point of the measurement library: the grid-wide
handoff with its work buffer in a static device array of the library
(qbd_grid_handoff_noalloc), against the same handoff over a caller
workspace (qbd_grid_handoff).  Two calls in a row, the second with fewer
phases, so the second starts from what the first left in the array: each
must report no wait given up and no value read back wrong, and return the
same last vector as the workspace call."""
import ctypes

import numpy as np
import pytest
import torch

from test_abi import ceiling_lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_handoff_matches_workspace(mode):
    lib = ceiling_lib()
    words = int(lib.qbd_grid_handoff_work_words())
    rwords = int(lib.qbd_grid_handoff_noalloc_result_words())
    work = torch.full((words + 64,), -1, dtype=torch.int32, device="cuda")
    off = (-work.data_ptr()) % 256 // 4
    result = torch.full((rwords,), -1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for phases in (37, 5):
        print(f"grid_handoff_noalloc mode={mode} phases={phases}", flush=True)
        assert lib.qbd_grid_handoff(mode, phases, work.data_ptr() + 4 * off, stream) == 0
        assert lib.qbd_grid_handoff_noalloc(mode, phases, result.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        w = work[off:off + words].cpu().numpy().view(np.uint32)
        r = result.cpu().numpy().view(np.uint32)
        assert w[words - 64] == 0 and w[words - 63] == 0, "workspace call"
        assert r[0] == 0, "a wait gave up"
        assert r[1] == 0, "vector values read back wrong"
        last = (phases - 1) & 1
        expect = np.arange(1024) * 7.0 + phases - 1
        ws_vec = w[1024 + last * 1024:1024 + (last + 1) * 1024].view(np.float32)
        na_vec = r[64:64 + 1024].view(np.float32)
        assert np.array_equal(ws_vec, expect)
        assert np.array_equal(na_vec, ws_vec)

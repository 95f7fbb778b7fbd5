"""The C ABI without a GPU: exported symbols, status codes, host validation
and the host-side block split helpers.

Validation runs before any HIP call, so every error path is reachable with
placeholder pointers.  Calls whose arguments pass validation would reach the
device; those are made only when no GPU is visible.
"""
import ctypes
import re

import numpy as np
import pytest
import torch

from block_quantized_decode_amd import binding

OK, NULL, SHAPE, ALIGN, ALIAS, DEVICE, LAUNCH = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(binding.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("qmv_q8_0_f32", "quantize_act_q8_0", "qmm_q8_0_q8act", "gate_up_swiglu_q4"):
        assert want in names
    assert sorted(names) == sorted(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = binding.lib()
    assert lib.qbd_abi_version() == 1
    for st in (OK, NULL, SHAPE, ALIGN, ALIAS, DEVICE, LAUNCH):
        assert binding.status_str(st)
    assert binding.status_str(12345) == "unknown status"


P = ctypes.c_void_p
BASE = 1 << 32  # placeholder addresses, far apart and 256-byte aligned


def fake(i, off=0):
    return P(BASE * (i + 1) + off)


def no_gpu():
    return torch.cuda.device_count() == 0


def call(name, *args):
    return getattr(binding.lib(), name)(*args)


def qmv_args(M=1, N=64, K=64, **over):
    a = dict(wq=fake(0), wd=fake(1), x=fake(2), y=fake(3), M=M, N=N, K=K)
    a.update(over)
    return [a["wq"], a["wd"], a["x"], a["y"], a["M"], a["N"], a["K"], P(0)]


@pytest.mark.parametrize("name", ["qmv_q8_0_f32", "qmv_q4_0_f32"])
def test_f32_validation(name):
    assert call(name, *qmv_args(K=48)) == SHAPE
    assert call(name, *qmv_args(K=0)) == SHAPE
    assert call(name, *qmv_args(K=-32)) == SHAPE
    assert call(name, *qmv_args(M=-1)) == SHAPE
    assert call(name, *qmv_args(N=-5)) == SHAPE
    assert call(name, *qmv_args(N=1 << 31)) == SHAPE
    assert call(name, *qmv_args(wq=P(0))) == NULL
    assert call(name, *qmv_args(wd=P(0))) == NULL
    assert call(name, *qmv_args(x=P(0))) == NULL
    assert call(name, *qmv_args(y=P(0))) == NULL
    assert call(name, *qmv_args(wq=fake(0, 8))) == ALIGN
    assert call(name, *qmv_args(wd=fake(1, 1))) == ALIGN
    assert call(name, *qmv_args(x=fake(2, 4))) == ALIGN
    assert call(name, *qmv_args(y=fake(3, 2))) == ALIGN
    assert call(name, *qmv_args(y=fake(0, 16))) == ALIAS       # y inside the codes
    assert call(name, *qmv_args(y=fake(2, 64))) == ALIAS       # y inside x (M*K*4 bytes)
    # nothing to do: no pointer is looked at
    assert call(name, *qmv_args(M=0, wq=P(0), x=P(0))) == OK
    assert call(name, *qmv_args(N=0, y=P(0))) == OK


def test_q8act_validation():
    def args(**over):
        a = dict(wq=fake(0), wd=fake(1), xq=fake(2), xd=fake(3), y=fake(4), M=2, N=8, K=64)
        a.update(over)
        return [a["wq"], a["wd"], a["xq"], a["xd"], a["y"], a["M"], a["N"], a["K"], P(0)]
    for name in ("qmm_q8_0_q8act", "qmm_q4_0_q8act"):
        assert call(name, *args(K=40)) == SHAPE
        assert call(name, *args(xd=P(0))) == NULL
        assert call(name, *args(xd=fake(3, 2))) == ALIGN
        assert call(name, *args(xq=fake(2, 4))) == ALIGN
        assert call(name, *args(y=fake(3, 4))) == ALIAS
        assert call(name, *args(y=fake(2))) == ALIAS
        assert call(name, *args(M=0)) == OK


def test_fused_validation():
    def args(**over):
        a = dict(gq=fake(0), gd=fake(1), uq=fake(2), ud=fake(3), x=fake(4), out=fake(5),
                 M=8, N=16, K=64)
        a.update(over)
        return [a["gq"], a["gd"], a["uq"], a["ud"], a["x"], a["out"], a["M"], a["N"], a["K"], P(0)]
    name = "gate_up_swiglu_q4"
    assert call(name, *args(uq=P(0))) == NULL
    assert call(name, *args(ud=P(0))) == NULL
    assert call(name, *args(uq=fake(2, 8))) == ALIGN
    assert call(name, *args(out=fake(2))) == ALIAS     # out over the up codes
    assert call(name, *args(out=fake(3))) == ALIAS     # out over the up scales
    assert call(name, *args(K=33)) == SHAPE

    def args8(**over):
        a = dict(gq=fake(0), gd=fake(1), uq=fake(2), ud=fake(3), xq=fake(4), xd=fake(5),
                 out=fake(6), M=8, N=16, K=64)
        a.update(over)
        return [a["gq"], a["gd"], a["uq"], a["ud"], a["xq"], a["xd"], a["out"], a["M"], a["N"],
                a["K"], P(0)]
    name = "gate_up_swiglu_q8_0"
    assert call(name, *args(gq=P(0))) == NULL
    assert call(name, *args(gd=fake(1, 1))) == ALIGN
    assert call(name, *args(x=fake(4, 4))) == ALIGN
    assert call(name, *args(out=fake(4, 32))) == ALIAS  # out over x
    assert call(name, *args(K=96 + 1)) == SHAPE
    assert call(name, *args(M=0, gq=P(0))) == OK

    name = "gate_up_swiglu_q4_q8act"
    assert call(name, *args8(xd=P(0))) == NULL
    assert call(name, *args8(out=fake(5))) == ALIAS
    assert call(name, *args8(N=0)) == OK


def test_from_f32_validation():
    # quantize + product in one call: x in, xq / xd / y out
    def args(**over):
        a = dict(wq=fake(0), wd=fake(1), x=fake(2), xq=fake(3), xd=fake(4), y=fake(5), M=1, N=8, K=64)
        a.update(over)
        return [a["wq"], a["wd"], a["x"], a["xq"], a["xd"], a["y"], a["M"], a["N"], a["K"], P(0)]
    for name in ("qmm_q8_0_q8act_from_f32", "qmm_q4_0_q8act_from_f32"):
        assert call(name, *args(K=40)) == SHAPE
        assert call(name, *args(x=P(0))) == NULL
        assert call(name, *args(xq=P(0))) == NULL
        assert call(name, *args(xd=P(0))) == NULL
        assert call(name, *args(x=fake(2, 8))) == ALIGN
        assert call(name, *args(xq=fake(3, 8))) == ALIGN
        assert call(name, *args(xd=fake(4, 2))) == ALIGN
        assert call(name, *args(xq=fake(2))) == ALIAS          # xq over x
        assert call(name, *args(xd=fake(1))) == ALIAS          # xd over the weight scales
        assert call(name, *args(y=fake(3, 32))) == ALIAS       # y over xq
        assert call(name, *args(xd=fake(3, 60))) == ALIAS      # xd over xq
        assert call(name, *args(M=0, x=P(0))) == OK
        assert call(name, *args(N=0, wq=P(0), x=P(0))) == NULL  # N = 0 still quantizes x

    def args2(**over):
        a = dict(gq=fake(0), gd=fake(1), uq=fake(2), ud=fake(3), x=fake(4), xq=fake(5), xd=fake(6),
                 out=fake(7), M=1, N=16, K=64)
        a.update(over)
        return [a["gq"], a["gd"], a["uq"], a["ud"], a["x"], a["xq"], a["xd"], a["out"], a["M"], a["N"],
                a["K"], P(0)]
    name = "gate_up_swiglu_q4_q8act_from_f32"
    assert call(name, *args2(uq=P(0))) == NULL
    assert call(name, *args2(ud=fake(3, 1))) == ALIGN
    assert call(name, *args2(out=fake(3))) == ALIAS           # out over the up scales
    assert call(name, *args2(xq=fake(2))) == ALIAS            # xq over the up codes
    assert call(name, *args2(M=0)) == OK


def test_quantize_and_swiglu_validation():
    q = "quantize_act_q8_0"
    assert call(q, fake(0), fake(1), fake(2), 4, 48, P(0)) == SHAPE
    assert call(q, P(0), fake(1), fake(2), 4, 64, P(0)) == NULL
    assert call(q, fake(0, 8), fake(1), fake(2), 4, 64, P(0)) == ALIGN
    assert call(q, fake(0), fake(1, 8), fake(2), 4, 64, P(0)) == ALIGN
    assert call(q, fake(0), fake(0, 512), fake(2), 4, 64, P(0)) == ALIAS   # xq over x
    assert call(q, fake(0), fake(1), fake(1, 64), 4, 64, P(0)) == ALIAS    # xd over xq
    assert call(q, fake(0), fake(1), fake(2), 0, 64, P(0)) == OK
    s = "swiglu_f32"
    assert call(s, fake(0), fake(1), fake(2), -1, P(0)) == SHAPE
    assert call(s, fake(0), P(0), fake(2), 8, P(0)) == NULL
    assert call(s, fake(0), fake(1), fake(2, 2), 8, P(0)) == ALIGN
    assert call(s, fake(0), fake(1), fake(1, 4), 8, P(0)) == ALIAS
    assert call(s, fake(0), fake(1), fake(2), 0, P(0)) == OK


@pytest.mark.skipif(not no_gpu(), reason="valid arguments would reach a real GPU")
def test_valid_arguments_reach_the_device_check():
    assert call("qmv_q8_0_f32", *qmv_args()) == DEVICE
    assert call("swiglu_f32", fake(0), fake(1), fake(2), 8, P(0)) == DEVICE


def test_binding_rejects_cpu_tensors():
    w = torch.zeros((4, 32), dtype=torch.int8)
    d = torch.zeros((4, 1), dtype=torch.int16)
    x = torch.zeros((1, 32), dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.qmv_q8_0_f32(w, d, x)
    with pytest.raises(TypeError):
        binding.qmv_q8_0_f32(w.to(torch.int16), d, x)


def test_split_blocks_q8():
    rng = np.random.default_rng(3)
    n, k = 5, 96
    codes = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    scales = rng.integers(0, 1 << 16, size=(n, k // 32), dtype=np.uint16)
    blocks = bytearray()
    for r in range(n):
        for b in range(k // 32):
            blocks += int(scales[r, b]).to_bytes(2, "little")
            blocks += codes[r, 32 * b:32 * b + 32].tobytes()
    wq, wd = binding.q8_0_split_blocks(bytes(blocks), n, k)
    assert np.array_equal(wq, codes) and np.array_equal(wd, scales)


def test_split_blocks_q4():
    rng = np.random.default_rng(4)
    n, k = 3, 64
    plane = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=(n, k // 32), dtype=np.uint16)
    blocks = bytearray()
    for r in range(n):
        for b in range(k // 32):
            blocks += int(scales[r, b]).to_bytes(2, "little")
            blocks += plane[r, 16 * b:16 * b + 16].tobytes()
    wq4, wd = binding.q4_0_split_blocks(bytes(blocks), n, k)
    assert np.array_equal(wq4, plane) and np.array_equal(wd, scales)
    assert call("q4_0_split_blocks", fake(0), fake(1), fake(2), 3, 40) == SHAPE
    assert call("q8_0_split_blocks", P(0), fake(1), fake(2), 3, 64) == NULL


def ceiling_lib():
    from block_quantized_decode_amd import build
    lib = ctypes.CDLL(build.CEILING_LIB)
    lib.qbd_read_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qbd_read_ceiling.restype = ctypes.c_int
    lib.qbd_read_ceiling_sink_words.restype = ctypes.c_int64
    lib.qbd_grid_handoff.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.qbd_grid_handoff.restype = ctypes.c_int
    lib.qbd_grid_handoff_work_words.restype = ctypes.c_int64
    lib.qbd_grid_handoff_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.qbd_grid_handoff_noalloc.restype = ctypes.c_int
    lib.qbd_grid_handoff_noalloc_result_words.restype = ctypes.c_int64
    lib.qbd_empty_launch.argtypes = [ctypes.c_void_p]
    lib.qbd_empty_launch.restype = ctypes.c_int
    return lib


def test_read_ceiling_library_exports_its_header():
    import os
    text = open(os.path.join(os.path.dirname(binding.HEADER_PATH), "qbd_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M))
    assert names == {"qbd_read_ceiling", "qbd_read_ceiling_sink_words", "qbd_grid_handoff",
                     "qbd_grid_handoff_work_words", "qbd_grid_handoff_noalloc",
                     "qbd_grid_handoff_noalloc_result_words", "qbd_empty_launch"}
    lib = ceiling_lib()
    for name in names:
        assert hasattr(lib, name), name
    assert lib.qbd_read_ceiling_sink_words() == 256 * 1024
    # arrival words, two 1024-float vectors, then the error words
    assert lib.qbd_grid_handoff_work_words() == 1024 + 2 * 1024 + 64
    # error words, then the last vector
    assert lib.qbd_grid_handoff_noalloc_result_words() == 64 + 1024


def test_read_ceiling_validation():
    # rejected before any HIP call
    lib = ceiling_lib()
    p = 1 << 20
    assert lib.qbd_read_ceiling(None, 64, p, None) == NULL
    assert lib.qbd_read_ceiling(p, 64, None, None) == NULL
    for bad in (0, -16, 8, 24):
        assert lib.qbd_read_ceiling(p, bad, p, None) == SHAPE
    assert lib.qbd_read_ceiling(p + 8, 64, p, None) == ALIGN
    assert lib.qbd_read_ceiling(p, 64, p + 2, None) == ALIGN


def test_grid_handoff_validation():
    # rejected before any HIP call
    lib = ceiling_lib()
    p = 1 << 20
    assert lib.qbd_grid_handoff(0, 1, None, None) == NULL
    for mode in (-1, 3):
        assert lib.qbd_grid_handoff(mode, 1, p, None) == SHAPE
    for phases in (-1, (1 << 20) + 1):
        assert lib.qbd_grid_handoff(0, phases, p, None) == SHAPE
    assert lib.qbd_grid_handoff(1, 1, p + 64, None) == ALIGN


def test_grid_handoff_noalloc_validation():
    # rejected before any HIP call
    lib = ceiling_lib()
    p = 1 << 20
    assert lib.qbd_grid_handoff_noalloc(0, 1, None, None) == NULL
    for mode in (-1, 3):
        assert lib.qbd_grid_handoff_noalloc(mode, 1, p, None) == SHAPE
    for phases in (-1, (1 << 20) + 1):
        assert lib.qbd_grid_handoff_noalloc(0, phases, p, None) == SHAPE
    assert lib.qbd_grid_handoff_noalloc(1, 1, p + 2, None) == ALIGN

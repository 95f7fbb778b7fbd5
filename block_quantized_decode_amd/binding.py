"""Python binding of libqbd: argument marshalling only.

Each function takes torch tensors on one gfx950 device, checks dtypes,
shapes, contiguity and that all tensors share that device, allocates the
output with torch when none is given, and calls the C entry point of the
same name with that device current, on torch's current stream for it.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback of any kind, and a missing library is an error.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqbd.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qbd.h")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64

# C signatures, mirrored from include/qbd.h
SIGNATURES = {
    "qbd_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "qbd_abi_version": ([], ctypes.c_int),
    "qmv_q8_0_f32": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "quantize_act_q8_0": ([_P, _P, _P, _I64, _I64, _P], ctypes.c_int),
    "qmm_q8_0_q8act": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "gate_up_swiglu_q4": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "gate_up_swiglu_q8_0": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmv_q4_0_f32": ([_P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmm_q4_0_q8act": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "gate_up_swiglu_q4_q8act": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmm_q8_0_q8act_from_f32": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "qmm_q4_0_q8act_from_f32": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "gate_up_swiglu_q4_q8act_from_f32": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "swiglu_f32": ([_P, _P, _P, _I64, _P], ctypes.c_int),
    "q8_0_split_blocks": ([_P, _P, _P, _I64, _I64], ctypes.c_int),
    "q4_0_split_blocks": ([_P, _P, _P, _I64, _I64], ctypes.c_int),
}

_lib = None


class QbdError(RuntimeError):
    """A libqbd entry point returned a non-zero status."""

    def __init__(self, name, status, text):
        super().__init__(f"{name}: {text} (status {status})")
        self.status = status


def lib():
    """Load libqbd.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_quantized_decode_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def status_str(status):
    return lib().qbd_status_str(int(status)).decode()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise QbdError(name, st, status_str(st))


def _launch(name, tensors, *args):
    """Call entry point `name` with the tensors' device current (the library
    checks and launches on the current device); every tensor must be on it."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"{name}: tensors on {dev} and {t.device}")
    with torch.cuda.device(dev):
        _call(name, *args, _stream(dev))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_I8 = (torch.int8,)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_SCALE = (torch.uint16, torch.int16)  # binary16 bit patterns


def _out(out, shape, dtype, like, name="out"):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _need(out, name, (dtype,), len(shape))
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def _weights(wq, wd, q4):
    _need(wq, "weight codes", _U8 if q4 else _I8, 2)
    _need(wd, "weight scales", _SCALE, 2)
    n = wq.shape[0]
    k = wq.shape[1] * (2 if q4 else 1)
    if tuple(wd.shape) != (n, k // 32) or k % 32:
        raise ValueError(f"weight planes {tuple(wq.shape)} / {tuple(wd.shape)} do not form [N][K]")
    return n, k


def qmv_q8_0_f32(wq, wd, x, out=None):
    """y[M][N] = x . W^T for Q8_0 weights (wq int8 [N][K], wd [N][K/32]) and fp32 x [M][K]."""
    n, k = _weights(wq, wd, False)
    _need(x, "x", _F32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x width differs from K")
    y = _out(out, (m, n), torch.float32, x)
    _launch("qmv_q8_0_f32", (x, wq, wd, y), _ptr(wq), _ptr(wd), _ptr(x), _ptr(y), m, n, k)
    return y


def qmv_q4_0_f32(wq4, wd, x, out=None):
    """y[M][N] = x . W^T for Q4 weights (wq4 uint8 [N][K/2], wd [N][K/32]) and fp32 x."""
    n, k = _weights(wq4, wd, True)
    _need(x, "x", _F32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x width differs from K")
    y = _out(out, (m, n), torch.float32, x)
    _launch("qmv_q4_0_f32", (x, wq4, wd, y), _ptr(wq4), _ptr(wd), _ptr(x), _ptr(y), m, n, k)
    return y


def gate_up_swiglu_q4(gq, gd, uq, ud, x, out=None):
    """out = silu(x . Wg^T) * (x . Wu^T), Q4 gate/up weights, fp32 x, one launch."""
    n, k = _weights(gq, gd, True)
    n2, k2 = _weights(uq, ud, True)
    if (n, k) != (n2, k2):
        raise ValueError("gate and up weights differ in shape")
    _need(x, "x", _F32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x width differs from K")
    o = _out(out, (m, n), torch.float32, x)
    _launch("gate_up_swiglu_q4", (x, gq, gd, uq, ud, o), _ptr(gq), _ptr(gd), _ptr(uq), _ptr(ud),
            _ptr(x), _ptr(o), m, n, k)
    return o


def gate_up_swiglu_q8_0(gq, gd, uq, ud, x, out=None):
    """out = silu(x . Wg^T) * (x . Wu^T), Q8_0 gate/up weights, fp32 x, one launch."""
    n, k = _weights(gq, gd, False)
    n2, k2 = _weights(uq, ud, False)
    if (n, k) != (n2, k2):
        raise ValueError("gate and up weights differ in shape")
    _need(x, "x", _F32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x width differs from K")
    o = _out(out, (m, n), torch.float32, x)
    _launch("gate_up_swiglu_q8_0", (x, gq, gd, uq, ud, o), _ptr(gq), _ptr(gd), _ptr(uq), _ptr(ud),
            _ptr(x), _ptr(o), m, n, k)
    return o


def quantize_act_q8_0(x, xq=None, xd=None):
    """Per-32-block Q8 quantization of fp32 x [M][K] -> (xq int8 [M][K], xd fp32 [M][K/32])."""
    _need(x, "x", _F32, 2)
    m, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    q = _out(xq, (m, k), torch.int8, x, "xq")
    d = _out(xd, (m, k // 32), torch.float32, x, "xd")
    _launch("quantize_act_q8_0", (x, q, d), _ptr(x), _ptr(q), _ptr(d), m, k)
    return q, d


def _act_q8(xq, xd, k):
    _need(xq, "xq", _I8, 2)
    _need(xd, "xd", _F32, 2)
    m = xq.shape[0]
    if xq.shape[1] != k or tuple(xd.shape) != (m, k // 32):
        raise ValueError("activation planes do not match K")
    return m


def qmm_q8_0_q8act(wq, wd, xq, xd, out=None):
    """y = sum_b d_w d_x dot_b for Q8_0 weights and Q8 activations (xq, xd)."""
    n, k = _weights(wq, wd, False)
    m = _act_q8(xq, xd, k)
    y = _out(out, (m, n), torch.float32, xq)
    _launch("qmm_q8_0_q8act", (xq, xd, wq, wd, y), _ptr(wq), _ptr(wd), _ptr(xq), _ptr(xd), _ptr(y),
            m, n, k)
    return y


def qmm_q4_0_q8act(wq4, wd, xq, xd, out=None):
    """y = sum_b d_w d_x dot_b for Q4 weights and Q8 activations (xq, xd)."""
    n, k = _weights(wq4, wd, True)
    m = _act_q8(xq, xd, k)
    y = _out(out, (m, n), torch.float32, xq)
    _launch("qmm_q4_0_q8act", (xq, xd, wq4, wd, y), _ptr(wq4), _ptr(wd), _ptr(xq), _ptr(xd), _ptr(y),
            m, n, k)
    return y


def gate_up_swiglu_q4_q8act(gq, gd, uq, ud, xq, xd, out=None):
    """out = silu(g) * u with g, u the Q4 x Q8-activation products, one launch."""
    n, k = _weights(gq, gd, True)
    n2, k2 = _weights(uq, ud, True)
    if (n, k) != (n2, k2):
        raise ValueError("gate and up weights differ in shape")
    m = _act_q8(xq, xd, k)
    o = _out(out, (m, n), torch.float32, xq)
    _launch("gate_up_swiglu_q4_q8act", (xq, xd, gq, gd, uq, ud, o), _ptr(gq), _ptr(gd), _ptr(uq),
            _ptr(ud), _ptr(xq), _ptr(xd), _ptr(o), m, n, k)
    return o


def _x_panel(x, k, xq, xd):
    _need(x, "x", _F32, 2)
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x width differs from K")
    return m, _out(xq, (m, k), torch.int8, x, "xq"), _out(xd, (m, k // 32), torch.float32, x, "xd")


def qmm_q8_0_q8act_from_f32(wq, wd, x, xq=None, xd=None, out=None):
    """quantize_act_q8_0(x) then qmm_q8_0_q8act in one call -> (y, xq, xd)."""
    n, k = _weights(wq, wd, False)
    m, q, d = _x_panel(x, k, xq, xd)
    y = _out(out, (m, n), torch.float32, x)
    _launch("qmm_q8_0_q8act_from_f32", (x, q, d, wq, wd, y), _ptr(wq), _ptr(wd), _ptr(x), _ptr(q), _ptr(d),
            _ptr(y), m, n, k)
    return y, q, d


def qmm_q4_0_q8act_from_f32(wq4, wd, x, xq=None, xd=None, out=None):
    """quantize_act_q8_0(x) then qmm_q4_0_q8act in one call -> (y, xq, xd)."""
    n, k = _weights(wq4, wd, True)
    m, q, d = _x_panel(x, k, xq, xd)
    y = _out(out, (m, n), torch.float32, x)
    _launch("qmm_q4_0_q8act_from_f32", (x, q, d, wq4, wd, y), _ptr(wq4), _ptr(wd), _ptr(x), _ptr(q), _ptr(d),
            _ptr(y), m, n, k)
    return y, q, d


def gate_up_swiglu_q4_q8act_from_f32(gq, gd, uq, ud, x, xq=None, xd=None, out=None):
    """quantize_act_q8_0(x) then gate_up_swiglu_q4_q8act in one call -> (out, xq, xd)."""
    n, k = _weights(gq, gd, True)
    n2, k2 = _weights(uq, ud, True)
    if (n, k) != (n2, k2):
        raise ValueError("gate and up weights differ in shape")
    m, q, d = _x_panel(x, k, xq, xd)
    o = _out(out, (m, n), torch.float32, x)
    _launch("gate_up_swiglu_q4_q8act_from_f32", (x, q, d, gq, gd, uq, ud, o), _ptr(gq), _ptr(gd), _ptr(uq),
            _ptr(ud), _ptr(x), _ptr(q), _ptr(d), _ptr(o), m, n, k)
    return o, q, d


def swiglu_f32(g, u, out=None):
    """out = silu(g) * u elementwise (fp32, same shape)."""
    if not isinstance(g, torch.Tensor) or not isinstance(u, torch.Tensor):
        raise TypeError("g and u must be tensors")
    if g.shape != u.shape or g.dtype != torch.float32 or u.dtype != torch.float32:
        raise ValueError("g and u must be fp32 tensors of one shape")
    if not (g.is_cuda and u.is_cuda and g.is_contiguous() and u.is_contiguous()):
        raise ValueError("g and u must be contiguous GPU tensors")
    o = torch.empty_like(g) if out is None else out
    if o.shape != g.shape or o.dtype != torch.float32 or not o.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like g")
    _launch("swiglu_f32", (g, u, o), _ptr(g), _ptr(u), _ptr(o), g.numel())
    return o


def q8_0_split_blocks(blocks34, n, k):
    """Host helper: interleaved 34-byte Q8_0 blocks (bytes) -> (wq, wd) numpy planes."""
    import numpy as np
    src = np.ascontiguousarray(np.frombuffer(blocks34, dtype=np.uint8))
    wq = np.empty((n, k), dtype=np.int8)
    wd = np.empty((n, k // 32), dtype=np.uint16)
    if src.size != n * (k // 32) * 34:
        raise ValueError("blocks34 size does not match N, K")
    _call("q8_0_split_blocks", src.ctypes.data_as(_P), wq.ctypes.data_as(_P),
          wd.ctypes.data_as(_P), n, k)
    return wq, wd


def q4_0_split_blocks(blocks18, n, k):
    """Host helper: interleaved 18-byte Q4 blocks (bytes) -> (wq4, wd) numpy planes."""
    import numpy as np
    src = np.ascontiguousarray(np.frombuffer(blocks18, dtype=np.uint8))
    wq4 = np.empty((n, k // 2), dtype=np.uint8)
    wd = np.empty((n, k // 32), dtype=np.uint16)
    if src.size != n * (k // 32) * 18:
        raise ValueError("blocks18 size does not match N, K")
    _call("q4_0_split_blocks", src.ctypes.data_as(_P), wq4.ctypes.data_as(_P),
          wd.ctypes.data_as(_P), n, k)
    return wq4, wd

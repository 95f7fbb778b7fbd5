"""Helpers of the GPU parity tests: device transfer, tolerance checks,
canary guards around outputs and input fingerprints."""
import hashlib
import sys

import numpy as np
import pytest
import torch

import oracle

CANARY = np.float32(-1.2345678e30)
PAD = 64  # guard elements on each side of an output


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(*parts):
    """Name the case on stdout before a GPU step (unbuffered)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_fp32(name, got, y64, s):
    """|got - y64| <= 1e-4 * S + 1e-6 elementwise."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == y64.shape, (name, got.shape, y64.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - y64)
    bound = oracle.fp32_bound(s)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} outputs out of bound; worst at {i}: "
                             f"got {got[i]!r} ref {y64[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")
    return float((err / bound).max()) if err.size else 0.0


def assert_swiglu(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    bound = oracle.swiglu_bound(ref["g64"], ref["u64"], ref["sg"], ref["su"])
    err = np.abs(got - ref["out64"])
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} outputs out of bound; worst at {i}: "
                             f"got {got[i]!r} ref {ref['out64'][i]!r} bound {bound[i]:.3e}")


CANARY_I8 = 91  # 0x5B


def _canary(dtype):
    return CANARY_I8 if dtype == torch.int8 else float(CANARY)


def guarded_out(shape, dtype=torch.float32):
    """An output view with PAD canary elements before and after it (PAD
    elements keep the view 64-byte aligned for 1-byte and 256-byte aligned
    for 4-byte elements)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * PAD,), _canary(dtype), dtype=dtype, device=device())
    return buf, buf[PAD:PAD + n].view(*shape)


def assert_guards(buf, name):
    b = host(buf)
    c = CANARY_I8 if b.dtype == np.int8 else CANARY
    assert np.all(b[:PAD] == c) and np.all(b[-PAD:] == c), f"{name}: wrote outside its output"


def fingerprint(*tensors):
    h = hashlib.sha256()
    for t in tensors:
        h.update(host(t).tobytes())
    return h.hexdigest()

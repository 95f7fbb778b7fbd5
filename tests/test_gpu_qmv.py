"""GPU parity: fp32-activation products (qmv_q8_0_f32, qmv_q4_0_f32) against
the oracle, through the C ABI."""
import numpy as np
import pytest

import block_quantized_decode_amd as qbd
from block_quantized_decode_amd import datagen
import oracle
from exact import pack_q4
from gpu_util import (assert_fp32, assert_guards, fingerprint, gpu, guarded_out, host, note)

pytestmark = pytest.mark.gpu

ONE_F16 = 0x3C00


def q8_case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    x = rng.standard_normal((m, k)).astype(np.float32)
    return wq, wd, x


def q4_case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    x = rng.standard_normal((m, k)).astype(np.float32)
    return wq, wd, x


SHAPES = [(1, 1, 32), (1, 5, 64), (1, 17, 96), (1, 64, 896), (1, 130, 1056), (1, 33, 4864),
          (1, 4100, 896), (1, 40000, 64), (1, 7, 8192),
          # many rows at M=1: the persistent grid, odd row counts and a tail
          # of clamped row groups
          (1, 40001, 96), (1, 65539, 32), (1, 70001, 896), (1, 9, 8224), (1, 3, 16384),
          # long rows at M=1 and few of them: one wave per K sweep, one or two
          # rows per workgroup (odd row counts), ragged last sweep, 16 sweeps
          (1, 896, 4864), (1, 2049, 4096), (1, 4095, 2080), (1, 300, 16384),
          (2, 17, 96), (3, 64, 896), (5, 33, 1056), (8, 130, 5120), (17, 9, 64), (33, 5, 128),
          # long rows at M=1 with x staged in LDS (ragged last sweep, LDS up to 70 KB)
          (1, 4100, 4864), (1, 4096, 2080), (1, 4500, 17408),
          # panels too long for LDS: x streamed in chunks of K (ragged last chunk)
          (2, 33, 10272), (8, 70, 5152), (5, 300, 17408), (7, 600, 12320),
          # panels of 2-16 rows over many 16-row tiles, on either side of the
          # matrix-core rule (9-16 rows; 4-bit weights with two tiles per CU):
          # ragged last tile, a partial last group of 4-bit blocks, panel
          # rows past M, up to 6 tiles per workgroup, more workgroups than CUs
          (2, 4096, 1024), (8, 4100, 1088), (5, 4111, 1152), (16, 4200, 2048), (9, 4097, 1024),
          (3, 12300, 1024), (2, 24580, 1024), (8, 4080, 1024), (8, 8200, 1088),
          # the most tiles per workgroup: six for panels of up to 8 rows, five
          # for 9-16 rows (N past 20480 on 256 CUs), ragged last tile
          (8, 24592, 1024), (12, 24592, 1024), (16, 20800, 1088), (9, 24600, 1024)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_qmv_q8_0_sweep(m, n, k):
    note("qmv_q8_0_f32 sweep", m, n, k)
    wq, wd, x = q8_case(100 + m * 7 + n + k, m, n, k)
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
    _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
    assert_fp32("qmv_q8_0_f32", y, y64, s)


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_qmv_q4_0_sweep(m, n, k):
    note("qmv_q4_0_f32 sweep", m, n, k)
    wq, wd, x = q4_case(200 + m * 7 + n + k, m, n, k)
    y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x)))
    _, y64, s = oracle.qmv_q4_0_f32(wq, wd, x)
    assert_fp32("qmv_q4_0_f32", y, y64, s)


@pytest.mark.parametrize("m,k", [(1, 896), (1, 4864), (3, 96), (1, 16384)])
def test_qmv_q8_0_one_hot_exact(m, k):
    """x = e_k selects d[n, k/32] * q[n, k] exactly."""
    n = 37
    wq, wd, _ = q8_case(5, 1, n, k)
    cols = [0, 31, 32, k // 2 + 5, k - 1][:m] if m > 1 else [k - 1]
    x = np.zeros((m, k), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    note("qmv_q8_0_f32 one-hot", m, k)
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
    want = np.stack([(oracle.fp16_bits_to_f64(wd[:, c // 32]) * wq[:, c]).astype(np.float32)
                     for c in cols])
    assert np.array_equal(y, want)


def test_qmv_q8_0_unit_scale_integers_exact():
    m, n, k = 3, 200, 4864
    rng = np.random.default_rng(9)
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    xi = rng.integers(-2, 3, size=(m, k))
    note("qmv_q8_0_f32 unit scale", m, n, k)
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(xi.astype(np.float32))))
    assert np.array_equal(y, (xi @ wq.astype(np.int64).T).astype(np.float32))


@pytest.mark.parametrize("n", [70, 4200])
def test_qmv_q4_all_eight_is_exactly_zero(n):
    m, k = 2, 5120
    rng = np.random.default_rng(10)
    wq = np.full((n, k // 2), 0x88, dtype=np.uint8)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    x = rng.standard_normal((m, k)).astype(np.float32)
    for mm in (1, m):
        note("qmv_q4_0_f32 all-8", mm)
        y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x[:mm])))
        assert np.all(y == 0)


@pytest.mark.parametrize("n,k", [(21, 2048), (4096, 2048), (21, 4864)])  # per-row, persistent rows, one wave per sweep
def test_qmv_q4_one_hot_exact(n, k):
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(n, k))
    wq = pack_q4(codes)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    for c in (0, 15, 16, 31, 1000, k - 1):
        x = np.zeros((1, k), dtype=np.float32)
        x[0, c] = 1.0
        note("qmv_q4_0_f32 one-hot", n, k, c)
        y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x)))
        want = (oracle.fp16_bits_to_f64(wd[:, c // 32]) * (codes[:, c] - 8)).astype(np.float32)
        assert np.array_equal(y[0], want)


def test_qmv_q8_0_subnormal_scales_and_inputs():
    m, n, k = 2, 40, 896
    rng = np.random.default_rng(12)
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = rng.integers(1, 0x0400, size=(n, k // 32)).astype(np.uint16)   # subnormal fp16 scales
    x = (rng.standard_normal((m, k)) * 2.0 ** -120).astype(np.float32)  # near/below fp32 min normal
    note("qmv_q8_0_f32 subnormals")
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
    _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
    assert_fp32("qmv_q8_0_f32 subnormal", y, y64, s)


def test_qmv_guards_readonly_replay():
    m, n, k = 1, 1152, 896
    wq, wd, x = q8_case(13, m, n, k)
    gw, gd, gx = gpu(wq), gpu(wd), gpu(x)
    before = fingerprint(gw, gd, gx)
    buf, out = guarded_out((m, n))
    note("qmv_q8_0_f32 guards")
    qbd.qmv_q8_0_f32(gw, gd, gx, out=out)
    first = host(out).copy()
    qbd.qmv_q8_0_f32(gw, gd, gx, out=out)
    assert np.array_equal(first, host(out))
    assert_guards(buf, "qmv_q8_0_f32")
    assert fingerprint(gw, gd, gx) == before


def test_empty_calls_are_noops():
    import torch
    note("empty calls")
    x = gpu(np.zeros((0, 64), dtype=np.float32))
    wq, wd, _ = q8_case(1, 1, 4, 64)
    y = qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), x)
    assert tuple(y.shape) == (0, 4)
    torch.cuda.synchronize()


def test_single_gemv_full():
    """Single Q8_0 GEMV, M=1, N=K=896, seeded inputs."""
    wq, wd, x = datagen.single_gemv()
    note("qmv_q8_0_f32 single GEMV 896x896")
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
    _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
    assert_fp32("single GEMV", y, y64, s)


def test_decode_layer_full():
    """Qwen2.5-0.5B-shaped decode layer at M=1: qkv, wo, gate, up, down."""
    mats = datagen.decode_layer_weights(0)
    acts = datagen.decode_activations(1)
    for name, n, k in datagen.DECODE_LAYER:
        wq, wd = mats[name]
        x = acts[k]
        note("qmv_q8_0_f32 decode layer", name, n, k)
        y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
        _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
        assert_fp32(name, y, y64, s)


def test_lm_head_full_sampled_rows():
    """LM head 896 -> 151936 at M=1, full launch; rows checked on a sample."""
    wq, wd = datagen.lm_head_weights(0)
    x = datagen.decode_activations(1)[896]
    note("qmv_q8_0_f32 lm_head 151936x896")
    y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
    rng = np.random.default_rng(14)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(wq.shape[0] - 256, wq.shape[0]),
                                     rng.choice(wq.shape[0], 8192, replace=False)]))
    _, y64, s = oracle.qmv_q8_0_f32(wq[rows], wd[rows], x)
    assert_fp32("lm_head", y[:, rows], y64, s)
    assert np.all(np.isfinite(y))


def test_down_projection_m8_full_sampled():
    """M=8 Q4 down projection N=5120, K=17408 (x streamed in chunks of K):
    the full launch, checked on sampled output rows."""
    m, n, k = 8, 5120, 17408
    wq, wd, x = q4_case(31, m, n, k)
    note("qmv_q4_0_f32 down M=8 5120x17408")
    y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x)))
    rows = np.unique(np.concatenate([np.arange(40), np.arange(n - 40, n),
                                     np.random.default_rng(32).choice(n, 400, replace=False)]))
    _, y64, s = oracle.qmv_q4_0_f32(wq[rows], wd[rows], x)
    assert_fp32("down M=8", y[:, rows], y64, s)


# Shapes on either side of each dispatch boundary (x in VGPRs / staged in
# LDS / generic for M=1; resident / chunked panels), LDS use up to 160 KB.
BOUNDARY_SHAPES = [
    ("q8", 1, 4096, 39936),   # M=1 staged, 39 sweeps: the largest x that fits
    ("q8", 1, 4096, 39968),   # one chunk more: generic kernel
    ("q4", 1, 4096, 38912),   # 4-bit staged at its limit
    ("q4", 1, 4096, 38944),   # generic
    ("q8", 1, 8192, 4096),    # staged from K = 4096 (Q8_0)
    ("q8", 1, 8192, 4064),    # x in VGPRs
    ("q4", 1, 4095, 5120),    # N just below the staging threshold
    ("q4", 1, 4096, 2048),    # staged from K = 2048 (4-bit)
    ("q4", 1, 4096, 2016),    # x in VGPRs
    ("q8", 1, 4095, 4864),    # one wave per sweep: the most rows
    ("q8", 1, 4096, 4864),    # one row more: x in VGPRs
    ("q8", 1, 300, 16384),    # one wave per sweep: 16 sweeps
    ("q8", 1, 300, 16416),    # one chunk more: x staged in LDS
    ("q4", 1, 300, 8192),     # 4-bit, one wave per sweep: 4 sweeps
    ("q4", 1, 300, 8224),     # one chunk more: x staged in LDS
    ("q4", 4, 100, 10240),    # resident 4-row panel filling 160 KB
    ("q4", 4, 100, 10272),    # chunked
    ("q8", 8, 300, 5120),     # resident 8-row panel filling 160 KB
    ("q8", 8, 300, 5152),     # chunked
]


@pytest.mark.parametrize("fmt,m,n,k", BOUNDARY_SHAPES)
def test_dispatch_boundaries(fmt, m, n, k):
    note("dispatch boundary", fmt, m, n, k)
    if fmt == "q8":
        wq, wd, x = q8_case(700 + m + n + k, m, n, k)
        y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
        _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
    else:
        wq, wd, x = q4_case(800 + m + n + k, m, n, k)
        y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x)))
        _, y64, s = oracle.qmv_q4_0_f32(wq, wd, x)
    assert_fp32(f"boundary {fmt} {m}x{n}x{k}", y, y64, s)


def test_q4_ffn_decode_full():
    """The 4-bit FFN at M=1 at full size, as the benchmark launches it: the
    gate/up GEMV 5120 -> 17408 (sampled rows) and the down projection
    17408 -> 5120 (all rows)."""
    rng_rows = np.random.default_rng(33)
    (_, ng, kg), (_, nd, kd) = datagen.Q4_FFN[0], datagen.Q4_FFN[2]
    w = datagen.q4_ffn_weights(0)
    x, h = datagen.q4_ffn_activations(1)
    note("q4 ffn gate M=1 full")
    y = host(qbd.qmv_q4_0_f32(gpu(w["gate"][0]), gpu(w["gate"][1]), gpu(x)))
    rows = np.unique(np.concatenate([np.arange(32), np.arange(ng - 32, ng), rng_rows.choice(ng, 1024, replace=False)]))
    _, y64, s = oracle.qmv_q4_0_f32(w["gate"][0][rows], w["gate"][1][rows], x)
    assert_fp32("q4 ffn gate", y[:, rows], y64, s)
    note("q4 ffn down M=1 full")
    y = host(qbd.qmv_q4_0_f32(gpu(w["down"][0]), gpu(w["down"][1]), gpu(h)))
    _, y64, s = oracle.qmv_q4_0_f32(w["down"][0], w["down"][1], h)
    assert_fp32("q4 ffn down", y, y64, s)


# The matrix-core panel (panels of 9-16 rows, or 4-bit weights over at least
# two 16-row tiles per CU) splits each fp32 activation into three bf16 parts
# whose sum is exact.  With codes that are powers of two every product
# code * x is exact in fp32, so a one-hot activation must come out as the
# correctly rounded d * (q - 8) * x, and any part dropped by the split would
# show.  (For panels of up to 8 rows the middle parts are accumulated
# separately and added once at the end, which is exact only for unit
# scales; those cases use d = 1.)
POW2_Q4 = np.array([0, 4, 6, 7, 9, 10, 12])          # 16 (q - 8) = +-2^j
POW2_Q8 = np.array([-128, -64, -16, -2, -1, 1, 2, 8, 32, 64])


@pytest.mark.parametrize("fmt,m,n", [("q4", 8, 8200), ("q4", 12, 4100), ("q8", 12, 4100), ("q8", 16, 4111)])
def test_mfma_panel_exact_split_one_hot(fmt, m, n):
    k = 1024
    rng = np.random.default_rng(23 + m)
    if fmt == "q4":
        codes = rng.choice(POW2_Q4, size=(n, k))
        wq = pack_q4(codes)
        vals = codes - 8
    else:
        wq = rng.choice(POW2_Q8, size=(n, k)).astype(np.int8)
        vals = wq.astype(np.int64)
    if m <= 8:
        wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    else:
        wd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    cols = rng.choice(k, size=m, replace=False)
    x = np.zeros((m, k), dtype=np.float32)
    # full 24-bit significands over a wide exponent range: all three parts nonzero
    mant = (1 << 23) | rng.integers(1, 1 << 23, size=m)
    x[np.arange(m), cols] = (mant * np.exp2(rng.integers(-40, 40, size=m) - 23.0)).astype(np.float32)
    note("mfma panel exact split", fmt, m, n, k)
    fn = qbd.qmv_q4_0_f32 if fmt == "q4" else qbd.qmv_q8_0_f32
    y = host(fn(gpu(wq), gpu(wd), gpu(x)))
    d = oracle.fp16_bits_to_f64(wd[:, cols // 32])                       # [n, m]
    want = (d * vals[:, cols] * x[np.arange(m), cols].astype(np.float64)).T.astype(np.float32)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("fmt,m,n", [("q4", 8, 8200), ("q4", 16, 4100), ("q8", 10, 4100)])
def test_mfma_panel_wide_range_activations(fmt, m, n):
    """Activations spanning 2^-60 .. 2^60 inside blocks, against the oracle."""
    k = 1088
    rng = np.random.default_rng(31 + m)
    x = (rng.standard_normal((m, k)) * np.exp2(rng.integers(-60, 61, size=(m, k)))).astype(np.float32)
    if fmt == "q4":
        wq, wd, _ = q4_case(41 + m, 1, n, k)
        note("mfma panel wide range q4", m, n, k)
        y = host(qbd.qmv_q4_0_f32(gpu(wq), gpu(wd), gpu(x)))
        _, y64, s = oracle.qmv_q4_0_f32(wq, wd, x)
    else:
        wq, wd, _ = q8_case(41 + m, 1, n, k)
        note("mfma panel wide range q8", m, n, k)
        y = host(qbd.qmv_q8_0_f32(gpu(wq), gpu(wd), gpu(x)))
        _, y64, s = oracle.qmv_q8_0_f32(wq, wd, x)
    assert_fp32(fmt, y, y64, s)

"""GPU parity: activation quantization (bit-exact), the Q8-activation
products (exact int32 block dots), SwiGLU and fused == unfused."""
import json
import os

import numpy as np
import pytest

import block_quantized_decode_amd as qbd
from block_quantized_decode_amd import datagen
import oracle
from gpu_util import (assert_fp32, assert_guards, assert_swiglu, device, fingerprint, gpu, guarded_out,
                      host, note)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE_F16 = 0x3C00


# ------------------------------------------------------------- quantization
@pytest.mark.parametrize("m,k", [(1, 32), (1, 896), (3, 96), (32, 896), (32, 4864), (7, 5120),
                                 (1024, 5120)])
def test_quantize_bit_exact(m, k):
    rng = np.random.default_rng(300 + m + k)
    x = datagen.activations(rng, m, k, outliers=True)
    x[0, :32] = 0.0                                    # an all-zero block
    note("quantize_act_q8_0", m, k)
    q, d = qbd.quantize_act_q8_0(gpu(x))
    q_ref, d_ref = oracle.quantize_act_q8_0(x)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))


def test_quantize_golden_ties():
    cases = json.load(open(os.path.join(GOLDEN, "quant_ties.json")))["cases"]
    x = np.array([c["x"] for c in cases], dtype=np.float32)
    note("quantize_act_q8_0 golden ties")
    q, d = qbd.quantize_act_q8_0(gpu(x))
    assert host(q).tolist() == [c["q"] for c in cases]
    assert [float(v) for v in host(d)[:, 0]] == [c["d"][0] for c in cases]


def test_quantize_subnormal_and_wide_range():
    rng = np.random.default_rng(301)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[0] *= np.float32(2.0 ** -130)      # subnormal inputs: d is subnormal too
    x[1] *= np.float32(2.0 ** 100)
    x[2, ::3] = 0.0
    x[3] = np.float32(2.0 ** -149)       # smallest subnormal everywhere
    note("quantize_act_q8_0 subnormal")
    q, d = qbd.quantize_act_q8_0(gpu(x))
    q_ref, d_ref = oracle.quantize_act_q8_0(x)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))


# ------------------------------------------------------ Q8 x Q8 / Q4 x Q8
def q8act_inputs(seed, m, n, k, q4):
    rng = np.random.default_rng(seed)
    if q4:
        wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        wd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    else:
        wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
        wd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    x = datagen.activations(rng, m, k, outliers=True)
    xq, xd = oracle.quantize_act_q8_0(x)
    return wq, wd, xq, xd


SHAPES = [(1, 1, 32), (1, 17, 96), (1, 64, 896), (1, 33, 4864), (2, 17, 96), (3, 64, 896),
          (8, 130, 5120), (32, 96, 896), (33, 9, 64), (1, 5000, 128), (256, 48, 128),
          # short panels on the split-K matrix-core kernel (4 and 8 waves, 1 and 2 row tiles)
          (16, 40, 4864), (32, 1152, 896), (48, 33, 1024), (64, 200, 512), (17, 31, 224),
          # and just past its tile limit
          (32, 16384, 64),
          # the LDS-DMA panel kernel: ragged rows and columns, odd and single
          # stage counts (four blocks a stage), the 32-row configuration; and
          # the staged kernel for K that is not whole stages
          (130, 200, 1024), (96, 70, 384), (200, 33, 128), (32, 16384, 128), (100, 90, 1088),
          (20, 16400, 256),
          # either side of each dispatch boundary: 64 / 65 rows (split-K or
          # not), 32 / 33 rows with at least 512 tiles (the 32- and the
          # 128-row LDS-DMA configurations, here with 33 and 40 rows of 128 and
          # a ragged last column tile), 128 / 129 rows, K of 3 blocks (staged
          # kernel) and a long M=1 row set
          (64, 300, 256), (65, 300, 256), (33, 8192, 128), (40, 16416, 128), (128, 64, 4096),
          (129, 70, 96), (1, 16384, 4096),
          # 16 x 16 tiles (Q8_0, 8..64 rows): ragged rows and columns, K of
          # 3, 5 and 33 blocks (a partial last quad), the most quads per wave
          # (K = 8192) and one block past it, and either side of the tile limit
          (20, 100, 96), (45, 70, 160), (8, 64, 8192), (12, 48, 8224), (24, 2000, 1056),
          (64, 1000, 4864), (32, 4096, 256), (32, 4112, 256), (9, 17, 32),
          # M = 1 with the panel staged in LDS (N >= 4096): one sweep, whole
          # groups of sweeps, a partial last group (Q8_0 K = 17408: 17 sweeps
          # in groups of 6; 4-bit: 9 in groups of 5), ragged row counts
          (1, 4096, 32), (1, 4100, 4864), (1, 4097, 17408), (1, 6000, 5120), (1, 4099, 2080),
          # 2..8 rows: the panel staged in LDS (N >= 1024) at 2 rows or with
          # K past the 16 x 16 tiles' quads (otherwise the tiles): 2, 4 and 8
          # padded rows, one step, steps of two sweeps with a partial last
          # step (K = 17408: 9 or 17 sweeps), rows per workgroup below and at
          # the wave count, a ragged last workgroup; and the same row counts
          # on the tiles
          (2, 1024, 32), (3, 1500, 96), (4, 4864, 896), (5, 2000, 4864), (7, 4097, 2080),
          (8, 1030, 17408), (6, 1100, 64), (3, 1500, 8224), (7, 1100, 9216), (2, 4864, 5120),
          # 4-bit weights on the 16 x 16 tiles (8..16 rows): one and several
          # quads per wave, the most (K = 8192), a ragged last column tile
          (8, 1000, 5120), (16, 33, 8192), (11, 250, 96),
          # the persistent 16 x 16 tiles (8..16 rows, at least 2 tiles per CU):
          # 2 quads per wave with a one-block last quad, 3 and 5 quads, 6 for
          # Q8_0 (4-bit: the per-workgroup tiles), ragged last tile, and 2 or
          # 3 tiles per workgroup
          (8, 8192, 1056), (11, 8200, 4864), (16, 9000, 2080), (13, 8300, 6144)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_qmm_q8_0_sweep(m, n, k):
    wq, wd, xq, xd = q8act_inputs(400 + m + n + k, m, n, k, False)
    note("qmm_q8_0_q8act", m, n, k)
    y = host(qbd.qmm_q8_0_q8act(gpu(wq), gpu(wd), gpu(xq), gpu(xd)))
    _, y64, s, _ = oracle.qmm_q8_0_q8act(wq, wd, xq, xd)
    assert_fp32("qmm_q8_0_q8act", y, y64, s)


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_qmm_q4_0_sweep(m, n, k):
    wq, wd, xq, xd = q8act_inputs(500 + m + n + k, m, n, k, True)
    note("qmm_q4_0_q8act", m, n, k)
    y = host(qbd.qmm_q4_0_q8act(gpu(wq), gpu(wd), gpu(xq), gpu(xd)))
    _, y64, s, _ = oracle.qmm_q4_0_q8act(wq, wd, xq, xd)
    assert_fp32("qmm_q4_0_q8act", y, y64, s)


@pytest.mark.parametrize("q4", [False, True])
@pytest.mark.parametrize("m", [1, 8, 16, 32, 64, 128])
def test_int_block_dots_exact(q4, m):
    """Unit weight scales and activation blocks with max |x| = 127 make
    d_w = d_x = 1, so y is the plain sum of the int32 block dots: bitwise."""
    n, k = 150, 896
    rng = np.random.default_rng(600 + m)
    if q4:
        wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        codes = oracle.q4_codes(wq, k) - 8
    else:
        wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
        codes = wq.astype(np.int64)
    wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    xi = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    xi[:, ::32] = 127.0
    xq, xd = oracle.quantize_act_q8_0(xi)
    assert np.all(xd == 1.0)
    note("int block dots", q4, m)
    fn = qbd.qmm_q4_0_q8act if q4 else qbd.qmm_q8_0_q8act
    y = host(fn(gpu(wq), gpu(wd), gpu(xq), gpu(xd)))
    want = oracle.block_dots(codes, xq).sum(axis=2)
    assert np.array_equal(y, want.astype(np.float32))


@pytest.mark.parametrize("q4,m,k", [(False, 8, 2080), (True, 8, 2080), (True, 16, 4864), (False, 16, 1056)])
def test_int_block_dots_exact_persistent_tiles(q4, m, k):
    """The unit-scale check of test_int_block_dots_exact on the persistent
    16 x 16 tiles (N = 8200: 513 tiles, a ragged last one; K with a partial
    last quad or 5 quads per wave): y is the plain sum of the int32 block
    dots, bit for bit, so the 4-bit -8 offset folded into the products is
    exact."""
    n = 8200
    rng = np.random.default_rng(650 + m + k)
    if q4:
        wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        codes = oracle.q4_codes(wq, k) - 8
    else:
        wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
        codes = wq.astype(np.int64)
    wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    xi = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    xi[:, ::32] = 127.0
    xq, xd = oracle.quantize_act_q8_0(xi)
    assert np.all(xd == 1.0)
    note("int block dots persistent", q4, m, k)
    fn = qbd.qmm_q4_0_q8act if q4 else qbd.qmm_q8_0_q8act
    y = host(fn(gpu(wq), gpu(wd), gpu(xq), gpu(xd)))
    dots = oracle.block_dots(codes, xq)
    # every partial sum, in any order, is an integer below 2^24: exact in fp32
    assert np.abs(dots).sum(axis=2).max() < 2 ** 24
    assert np.array_equal(y, dots.sum(axis=2).astype(np.float32))


@pytest.mark.parametrize("q4,m,k", [(True, 8, 5120), (False, 12, 2080), (True, 16, 1056)])
def test_persistent_tiles_equal_tile_per_workgroup(q4, m, k):
    """N = 8192 takes the persistent 16 x 16 tiles (512 tiles, two per CU on
    256 CUs), N = 8176 one tile per workgroup (511 tiles): the first 8176
    outputs are bit for bit the same, plain and (4-bit) fused."""
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tile-count threshold is set for 256 CUs")
    rng = np.random.default_rng(660 + m + k)
    if q4:
        G = [datagen.q4_weights(rng, rng, 8192, k) for _ in range(2)]
    else:
        G = [datagen.q8_weights(rng, rng, 8192, k)]
    x = datagen.activations(rng, m, k, outliers=True)
    xq, xd = (gpu(a) for a in oracle.quantize_act_q8_0(x))
    fn = qbd.qmm_q4_0_q8act if q4 else qbd.qmm_q8_0_q8act
    note("persistent vs per-workgroup tiles", q4, m, k)
    wq, wd = G[0]
    big = host(fn(gpu(wq), gpu(wd), xq, xd))
    small = host(fn(gpu(wq[:8176]), gpu(wd[:8176]), xq, xd))
    assert np.array_equal(big[:, :8176].view(np.uint32), small.view(np.uint32))
    if q4:
        uq, ud = G[1]
        big = host(qbd.gate_up_swiglu_q4_q8act(gpu(wq), gpu(wd), gpu(uq), gpu(ud), xq, xd))
        small = host(qbd.gate_up_swiglu_q4_q8act(gpu(wq[:8176]), gpu(wd[:8176]), gpu(uq[:8176]), gpu(ud[:8176]),
                                                 xq, xd))
        assert np.array_equal(big[:, :8176].view(np.uint32), small.view(np.uint32))


def test_q8act_m1_decode_layer_shapes():
    """Q8 x Q8 path, decode-layer shapes at M=1 and M=32 (quantized on device)."""
    for m in (1, datagen.PP32_M):
        for name, n, k in datagen.DECODE_LAYER:
            wq, wd, x = datagen.q8q8_inputs(n, k, m)
            note("q8q8 decode layer", name, m)
            xq, xd = qbd.quantize_act_q8_0(gpu(x))
            q_ref, d_ref = oracle.quantize_act_q8_0(x)
            assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xd), d_ref)
            y = host(qbd.qmm_q8_0_q8act(gpu(wq), gpu(wd), xq, xd))
            _, y64, s, _ = oracle.qmm_q8_0_q8act(wq, wd, q_ref, d_ref)
            assert_fp32(f"q8q8 {name} M={m}", y, y64, s)


def test_q8act_lm_head_sampled():
    name, n, k = datagen.LM_HEAD
    for m in (1, datagen.PP32_M):
        wq, wd, x = datagen.q8q8_inputs(n, k, m)
        note("q8q8 lm_head", m)
        xq, xd = qbd.quantize_act_q8_0(gpu(x))
        y = host(qbd.qmm_q8_0_q8act(gpu(wq), gpu(wd), xq, xd))
        rows = np.random.default_rng(15).choice(n, 2048, replace=False)
        q_ref, d_ref = oracle.quantize_act_q8_0(x)
        _, y64, s, _ = oracle.qmm_q8_0_q8act(wq[rows], wd[rows], q_ref, d_ref)
        assert_fp32(f"q8q8 lm_head M={m}", y[:, rows], y64, s)


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_f32_elementwise():
    rng = np.random.default_rng(700)
    g = np.concatenate([rng.standard_normal(5000) * 6, [0.0, -0.0, -90.0, -200.0, 88.0, 1e-30,
                                                         -1e-30, 30.0, -30.0]]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32)
    note("swiglu_f32")
    out = host(qbd.swiglu_f32(gpu(g), gpu(u)))
    _, out64 = oracle.swiglu_f32(g, u)
    assert np.all(np.abs(out.astype(np.float64) - out64) <= oracle.swiglu_elementwise_bound(out64))


def gpu_scales_off4(wd):
    """The weight scales on the GPU at an address that is 2 mod 4 (allowed by
    the C ABI, which asks 2-byte alignment of scales): such a call takes the
    register-staged panel kernel instead of the LDS-copy one."""
    import torch
    flat = torch.zeros(wd.size + 1, dtype=torch.int16, device=device())
    view = flat[1:].view(wd.shape)
    view.copy_(gpu(wd.view(np.int16)))
    assert view.data_ptr() % 4 == 2
    return view


def gpu_act_scales_off4(xd):
    """The activation scales on the GPU at an address that is 4 mod 16 (the
    C ABI asks 4-byte alignment of scales).  The LDS-copy kernel copies the
    four scales of a row and stage as one 16-byte piece, so such a call takes
    the register-staged kernel."""
    import torch
    flat = torch.zeros(xd.size + 1, dtype=torch.float32, device=device())
    view = flat[1:].view(xd.shape)
    view.copy_(gpu(xd))
    assert view.data_ptr() % 16 == 4
    return view


@pytest.mark.parametrize("q4,m,n,k", [(True, 256, 200, 1024), (True, 130, 96, 384), (False, 130, 96, 384),
                                      (False, 300, 64, 2048), (True, 32, 16384, 128),
                                      # short panels (split-K kernel): scales at 2 mod 4 take the
                                      # same path and must give the same bits
                                      (False, 32, 1152, 896), (False, 16, 40, 4864), (True, 32, 96, 896),
                                      (False, 20, 100, 2112), (True, 32, 64, 64)])
def test_qmm_lds_copy_kernel_equals_staged_kernel(q4, m, n, k):
    """The panel kernel that copies stages straight into LDS and the one that
    stages them through registers form the same block dots, scaled and added
    in the same order: their outputs agree bitwise."""
    wq, wd, xq, xd = q8act_inputs(700 + m + n + k, m, n, k, q4)
    fn = qbd.qmm_q4_0_q8act if q4 else qbd.qmm_q8_0_q8act
    Wq, Xq, Xd = gpu(wq), gpu(xq), gpu(xd)
    note("LDS-copy vs staged panel kernel", q4, m, n, k)
    a = host(fn(Wq, gpu(wd), Xq, Xd))
    b = host(fn(Wq, gpu_scales_off4(wd), Xq, Xd))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = host(fn(Wq, gpu(wd), Xq, gpu_act_scales_off4(xd)))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    _, y64, s, _ = oracle.qmm_q4_0_q8act(wq, wd, xq, xd) if q4 else oracle.qmm_q8_0_q8act(wq, wd, xq, xd)
    assert_fp32("LDS-copy panel kernel", a, y64, s)


@pytest.mark.parametrize("m,n,k", [(200, 130, 1024), (32, 96, 896)])
def test_gate_up_q8act_lds_copy_kernel_equals_staged_kernel(m, n, k):
    gq, gd, uq, ud, x = q4_pair(760, m, n, k)
    xq, xd = oracle.quantize_act_q8_0(x)
    G = [gpu(a) for a in (gq, gd, uq, ud, xq, xd)]
    note("gate_up_swiglu_q4_q8act LDS-copy vs staged", m, n, k)
    a = host(qbd.gate_up_swiglu_q4_q8act(*G))
    b = host(qbd.gate_up_swiglu_q4_q8act(G[0], gpu_scales_off4(gd), G[2], G[3], G[4], G[5]))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = host(qbd.gate_up_swiglu_q4_q8act(*G[:5], gpu_act_scales_off4(xd)))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def q4_pair(seed, m, n, k):
    rng = np.random.default_rng(seed)
    gq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    uq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    gd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    ud = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
    x = rng.standard_normal((m, k)).astype(np.float32)
    return gq, gd, uq, ud, x


FUSED_SHAPES = [(1, 17, 96), (1, 200, 5120), (2, 33, 128), (3, 64, 896), (8, 130, 5120),
                (8, 1000, 1024), (16, 48, 2048), (20, 40, 256), (64, 96, 512),
                (1, 4100, 2080), (1, 4096, 5120), (8, 100, 6144), (3, 64, 10272),
                # M=1, one wave per K sweep (one and two rows per workgroup)
                (1, 896, 4864), (1, 2049, 4096),
                (1, 40001, 64), (8, 4100, 1088), (16, 4104, 1024), (2, 12300, 1024), (8, 8200, 1088),
                # matrix-core panels with six (8 rows) and five (9-16 rows) tiles per workgroup
                (8, 24592, 1024), (12, 24592, 1024), (16, 20800, 1088),
                # the persistent 16 x 16 tiles: 2, 3 and 5 quads per wave, ragged tiles
                (8, 8208, 1056), (12, 8704, 2080), (16, 8200, 4864),
                # 16 x 16 tiles at the most quads per wave, a ragged column tile
                (13, 1030, 8192)]


@pytest.mark.parametrize("m,n,k", FUSED_SHAPES)
def test_gate_up_swiglu_q4_fused_equals_unfused(m, n, k):
    gq, gd, uq, ud, x = q4_pair(800 + m + n + k, m, n, k)
    G = [gpu(a) for a in (gq, gd, uq, ud, x)]
    note("gate_up_swiglu_q4", m, n, k)
    fused = host(qbd.gate_up_swiglu_q4(*G))
    g = qbd.qmv_q4_0_f32(G[0], G[1], G[4])
    u = qbd.qmv_q4_0_f32(G[2], G[3], G[4])
    unfused = host(qbd.swiglu_f32(g, u))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    assert_swiglu("gate_up_swiglu_q4", fused, oracle.gate_up_swiglu_q4(gq, gd, uq, ud, x))


@pytest.mark.parametrize("m,n,k", FUSED_SHAPES + [(256, 64, 512), (1024, 32, 256), (130, 200, 1024),
                                                   (96, 70, 384), (32, 16384, 128), (100, 90, 1088),
                                                   # dispatch boundaries, as for the plain products
                                                   (65, 300, 256), (33, 8192, 128), (40, 16416, 128),
                                                   (129, 70, 96)])
def test_gate_up_swiglu_q4_q8act_fused_equals_unfused(m, n, k):
    gq, gd, uq, ud, x = q4_pair(900 + m + n + k, m, n, k)
    xq, xd = oracle.quantize_act_q8_0(x)
    G = [gpu(a) for a in (gq, gd, uq, ud, xq, xd)]
    note("gate_up_swiglu_q4_q8act", m, n, k)
    fused = host(qbd.gate_up_swiglu_q4_q8act(*G))
    g = qbd.qmm_q4_0_q8act(G[0], G[1], G[4], G[5])
    u = qbd.qmm_q4_0_q8act(G[2], G[3], G[4], G[5])
    unfused = host(qbd.swiglu_f32(g, u))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    assert_swiglu("gate_up_swiglu_q4_q8act", fused,
                  oracle.gate_up_swiglu_q4_q8act(gq, gd, uq, ud, xq, xd))


def q8_pair(seed, m, n, k):
    rng = np.random.default_rng(seed)
    gq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    uq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    gd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    ud = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    x = rng.standard_normal((m, k)).astype(np.float32)
    return gq, gd, uq, ud, x


# M=1 in VGPRs and staged in LDS, resident and chunked panels
Q8_FUSED_SHAPES = [(1, 17, 96), (1, 4864, 896), (1, 4100, 4864), (1, 896, 4864), (1, 2049, 4096),
                   (1, 300, 16384), (2, 33, 128), (8, 130, 5120),
                   (8, 70, 5152), (5, 64, 1024), (16, 48, 2048), (1, 40001, 96), (8, 4100, 1088),
                   (13, 4112, 1024), (12, 24592, 1024), (16, 20800, 1088)]


@pytest.mark.parametrize("m,n,k", Q8_FUSED_SHAPES)
def test_gate_up_swiglu_q8_0_fused_equals_unfused(m, n, k):
    gq, gd, uq, ud, x = q8_pair(1000 + m + n + k, m, n, k)
    G = [gpu(a) for a in (gq, gd, uq, ud, x)]
    note("gate_up_swiglu_q8_0", m, n, k)
    fused = host(qbd.gate_up_swiglu_q8_0(*G))
    g = qbd.qmv_q8_0_f32(G[0], G[1], G[4])
    u = qbd.qmv_q8_0_f32(G[2], G[3], G[4])
    unfused = host(qbd.swiglu_f32(g, u))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    assert_swiglu("gate_up_swiglu_q8_0", fused, oracle.gate_up_swiglu_q8_0(gq, gd, uq, ud, x))


def test_gate_up_full_size_sampled():
    """Fused gate/up SwiGLU at M=8, N=17408, K=5120; full launch, sampled rows."""
    gq, gd, uq, ud, x = datagen.gate_up_inputs()
    G = [gpu(a) for a in (gq, gd, uq, ud, x)]
    before = fingerprint(*G)
    buf, out = guarded_out((x.shape[0], gq.shape[0]))
    note("gate_up_swiglu_q4 full 8x17408x5120")
    qbd.gate_up_swiglu_q4(*G, out=out)
    got = host(out)
    assert_guards(buf, "gate_up_swiglu_q4")
    assert fingerprint(*G) == before
    rows = np.unique(np.concatenate([np.arange(64), np.arange(gq.shape[0] - 64, gq.shape[0]),
                                     np.random.default_rng(16).choice(gq.shape[0], 1024, replace=False)]))
    ref = oracle.gate_up_swiglu_q4(gq[rows], gd[rows], uq[rows], ud[rows], x)
    assert_swiglu("gate_up full", got[:, rows], ref)
    # the fused output equals the unfused composition everywhere
    g = qbd.qmv_q4_0_f32(G[0], G[1], G[4])
    u = qbd.qmv_q4_0_f32(G[2], G[3], G[4])
    assert np.array_equal(got.view(np.uint32), host(qbd.swiglu_f32(g, u)).view(np.uint32))


def test_prefill_full_size_sampled():
    """M=1024, N=17408, K=5120 Q4 x Q8 activations (quantized on device):
    plain and fused-SwiGLU launches at full size; outputs checked on sampled
    rows and columns."""
    gq, gd, uq, ud, x = datagen.prefill_inputs()
    note("prefill quantize 1024x5120")
    xq, xd = qbd.quantize_act_q8_0(gpu(x))
    q_ref, d_ref = oracle.quantize_act_q8_0(x)
    assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xd), d_ref)
    G = [gpu(a) for a in (gq, gd, uq, ud)]
    note("prefill qmm_q4_0_q8act 1024x17408x5120")
    y = host(qbd.qmm_q4_0_q8act(G[0], G[1], xq, xd))
    note("prefill gate_up_swiglu_q4_q8act 1024x17408x5120")
    out = host(qbd.gate_up_swiglu_q4_q8act(G[0], G[1], G[2], G[3], xq, xd))
    # all rows x 256 columns (about half of the 544 column tiles of 32), and
    # 16 full rows: two in each 128-row workgroup tile, in both 64-row halves
    rng = np.random.default_rng(17)
    cols = np.unique(np.concatenate([[0, gq.shape[0] - 1], rng.choice(gq.shape[0], 254, replace=False)]))
    _, y64, s, _ = oracle.qmm_q4_0_q8act(gq[cols], gd[cols], q_ref, d_ref)
    assert_fp32("prefill plain (all rows, sampled cols)", y[:, cols], y64, s)
    ref = oracle.gate_up_swiglu_q4_q8act(gq[cols], gd[cols], uq[cols], ud[cols], q_ref, d_ref)
    assert_swiglu("prefill fused (all rows, sampled cols)", out[:, cols], ref)
    rows = np.array([128 * t + o for t in range(8) for o in ((5 * t) % 64, 64 + (37 * t) % 64)])
    assert len(np.unique(rows)) == 16
    _, y64r, sr, _ = oracle.qmm_q4_0_q8act(gq, gd, q_ref[rows], d_ref[rows])
    assert_fp32("prefill plain (sampled rows, all cols)", y[rows], y64r, sr)
    ref_r = oracle.gate_up_swiglu_q4_q8act(gq, gd, uq, ud, q_ref[rows], d_ref[rows])
    assert_swiglu("prefill fused (sampled rows, all cols)", out[rows], ref_r)


def test_q4_ffn_gate_up_m1_full():
    """Fused 4-bit gate/up SwiGLU at M=1, N=17408, K=5120 (the benchmark's
    decode launch): sampled rows against the oracle, and every output equal
    to the unfused composition."""
    w = datagen.q4_ffn_weights(0)
    x, _ = datagen.q4_ffn_activations(1)
    G = [gpu(a) for a in (*w["gate"], *w["up"], x)]
    note("q4 ffn fused gate/up M=1 full")
    out = host(qbd.gate_up_swiglu_q4(*G))
    g = qbd.qmv_q4_0_f32(G[0], G[1], G[4])
    u = qbd.qmv_q4_0_f32(G[2], G[3], G[4])
    assert np.array_equal(out.view(np.uint32), host(qbd.swiglu_f32(g, u)).view(np.uint32))
    n = w["gate"][0].shape[0]
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(34).choice(n, 512, replace=False)]))
    ref = oracle.gate_up_swiglu_q4(w["gate"][0][rows], w["gate"][1][rows], w["up"][0][rows], w["up"][1][rows], x)
    assert_swiglu("q4 ffn fused gate/up M=1", out[:, rows], ref)


# Shapes whose one-matrix scale rows fit the matrix-core panel's LDS but
# whose two-matrix rows do not: the plain and the fused call must take the
# same (VALU panel) kernel and agree bitwise.
TWO_MATRIX_BUDGET_SHAPES = [("q4", 8, 24576, 16384), ("q8", 12, 24576, 16384), ("q4", 8, 8192, 40960)]


@pytest.mark.slow
@pytest.mark.parametrize("fmt,m,n,k", TWO_MATRIX_BUDGET_SHAPES)
def test_fused_equals_unfused_at_lds_budget_edge(fmt, m, n, k):
    rng = np.random.default_rng(1100 + m + n // 1024 + k // 1024)
    if fmt == "q4":
        gq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        uq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        gd = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
        ud = datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03)
        fused_fn, plain_fn, ref_fn = qbd.gate_up_swiglu_q4, qbd.qmv_q4_0_f32, oracle.gate_up_swiglu_q4
    else:
        gq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
        uq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
        gd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
        ud = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
        fused_fn, plain_fn, ref_fn = qbd.gate_up_swiglu_q8_0, qbd.qmv_q8_0_f32, oracle.gate_up_swiglu_q8_0
    x = rng.standard_normal((m, k)).astype(np.float32)
    G = [gpu(a) for a in (gq, gd, uq, ud, x)]
    note("fused == unfused at the two-matrix LDS budget", fmt, m, n, k)
    fused = host(fused_fn(*G))
    g = plain_fn(G[0], G[1], G[4])
    u = plain_fn(G[2], G[3], G[4])
    unfused = host(qbd.swiglu_f32(g, u))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), rng.choice(n, 48, replace=False)]))
    ref = ref_fn(gq[rows], gd[rows], uq[rows], ud[rows], x)
    assert_swiglu(f"fused {fmt} at the LDS budget edge", fused[:, rows], ref)


# Canary guards around the output, inputs unchanged (read-only) and a
# second call giving the same bits (replay), for each entry point and the
# prefill-sized launches (LSE v0.4.15 release page, "Qualification and
# measurements": guards, read-only inputs, replays).
GUARD_CASES = [("quantize", 1, 0, 896), ("quantize", 32, 0, 4864), ("quantize", 1024, 0, 5120),
               ("qmm_q8_0", 1, 1152, 896), ("qmm_q8_0", 32, 896, 4864), ("qmm_q8_0", 130, 200, 1024),
               ("qmm_q4_0", 32, 1152, 896), ("qmm_q4_0", 1024, 17408, 5120),
               ("gate_up_q4_q8act", 8, 130, 5120), ("gate_up_q4_q8act", 1024, 17408, 5120),
               ("qmv_q4_0", 8, 17408, 5120), ("gate_up_q4", 8, 17408, 5120), ("gate_up_q8_0", 1, 4864, 896),
               # M=1, one wave per K sweep (one and two rows per workgroup)
               ("qmv_q4_0", 1, 300, 4864), ("gate_up_q8_0", 1, 896, 4864),
               ("swiglu", 0, 5000, 0)]


@pytest.mark.parametrize("kind,m,n,k", GUARD_CASES)
def test_guards_readonly_replay(kind, m, n, k):
    import torch
    rng = np.random.default_rng(1200 + m + n + k)
    note("guards/read-only/replay", kind, m, n, k)
    if kind == "quantize":
        x = gpu(datagen.activations(rng, m, k, outliers=True))
        before = fingerprint(x)
        qbuf, xq = guarded_out((m, k), torch.int8)
        dbuf, xd = guarded_out((m, k // 32))
        qbd.quantize_act_q8_0(x, xq, xd)
        first = (host(xq).copy(), host(xd).copy())
        qbd.quantize_act_q8_0(x, xq, xd)
        assert np.array_equal(first[0], host(xq)) and np.array_equal(first[1].view(np.uint32), host(xd).view(np.uint32))
        assert_guards(qbuf, "quantize codes")
        assert_guards(dbuf, "quantize scales")
        assert fingerprint(x) == before
        q_ref, d_ref = oracle.quantize_act_q8_0(host(x))
        assert np.array_equal(first[0], q_ref)
        return
    if kind == "swiglu":
        g, u = gpu(rng.standard_normal(n).astype(np.float32)), gpu(rng.standard_normal(n).astype(np.float32))
        before = fingerprint(g, u)
        buf, out = guarded_out((n,))
        qbd.swiglu_f32(g, u, out=out)
        first = host(out).copy()
        qbd.swiglu_f32(g, u, out=out)
        assert np.array_equal(first.view(np.uint32), host(out).view(np.uint32))
        assert_guards(buf, "swiglu_f32")
        assert fingerprint(g, u) == before
        return
    q4 = kind in ("qmm_q4_0", "gate_up_q4_q8act", "qmv_q4_0", "gate_up_q4")
    two = kind.startswith("gate_up")
    if q4:
        w = [rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8) for _ in range(2)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03) for _ in range(2)]
    else:
        w = [rng.integers(-127, 128, size=(n, k), dtype=np.int8) for _ in range(2)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02) for _ in range(2)]
    W = [gpu(a) for a in (w[0], d[0], w[1], d[1])]
    x = datagen.activations(rng, m, k, outliers=True)
    if kind in ("qmv_q4_0", "gate_up_q4", "gate_up_q8_0"):
        A = [gpu(x)]
    else:
        xq, xd = oracle.quantize_act_q8_0(x)
        A = [gpu(xq), gpu(xd)]
    fn = {"qmm_q8_0": qbd.qmm_q8_0_q8act, "qmm_q4_0": qbd.qmm_q4_0_q8act,
          "gate_up_q4_q8act": qbd.gate_up_swiglu_q4_q8act, "qmv_q4_0": qbd.qmv_q4_0_f32,
          "gate_up_q4": qbd.gate_up_swiglu_q4, "gate_up_q8_0": qbd.gate_up_swiglu_q8_0}[kind]
    args = (W if two else W[:2]) + A
    before = fingerprint(*args)
    buf, out = guarded_out((m, n))
    fn(*args, out=out)
    first = host(out).copy()
    fn(*args, out=out)
    assert np.array_equal(first.view(np.uint32), host(out).view(np.uint32))
    assert_guards(buf, kind)
    assert fingerprint(*args) == before
    assert np.all(np.isfinite(first))


# ------------------------------------------- one activation producer, several consumers
@pytest.mark.parametrize("m", [1, 8, 32])
def test_shared_producer_feeds_four_consumers(m):
    """One quantize_act_q8_0 panel feeding the qkv, wo, gate and up products
    of the decode layer (one producer for four projections, LSE v0.4.15
    release page, "Changes"): the codes are bit-exact, every consumer
    matches the oracle, and each equals bitwise the same product fed by a
    producer of its own."""
    rng = np.random.default_rng(1600 + m)
    x = datagen.activations(rng, m, 896, outliers=True)
    X = gpu(x)
    note("shared producer", m)
    xq, xd = qbd.quantize_act_q8_0(X)
    q_ref, d_ref = oracle.quantize_act_q8_0(x)
    assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xd).view(np.uint32), d_ref.view(np.uint32))
    mats = datagen.decode_layer_weights(40)
    for name in ("qkv", "wo", "gate", "up"):
        wq, wd = mats[name]
        W, D = gpu(wq), gpu(wd)
        shared = host(qbd.qmm_q8_0_q8act(W, D, xq, xd))
        own_q, own_d = qbd.quantize_act_q8_0(X)
        own = host(qbd.qmm_q8_0_q8act(W, D, own_q, own_d))
        assert np.array_equal(shared.view(np.uint32), own.view(np.uint32)), name
        _, y64, s, _ = oracle.qmm_q8_0_q8act(wq, wd, q_ref, d_ref)
        assert_fp32(f"shared producer -> {name}", shared, y64, s)
    # the consumers leave the shared panel as the producer wrote it
    assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xd).view(np.uint32), d_ref.view(np.uint32))


def test_q4_ffn_q8act_m1_full():
    """The 4-bit FFN of the 27B-class target at M=1 on Q8 activations, as
    the benchmark launches it: quantize x, fused gate/up SwiGLU 5120 -> 17408
    (sampled rows against the oracle, all rows equal to the unfused
    composition), quantize h, down 17408 -> 5120 (all rows)."""
    w = datagen.q4_ffn_weights(0)
    x, h = datagen.q4_ffn_activations(1)
    note("q4 ffn q8act M=1: quantize x")
    xq, xd = qbd.quantize_act_q8_0(gpu(x))
    q_ref, d_ref = oracle.quantize_act_q8_0(x)
    assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xd).view(np.uint32), d_ref.view(np.uint32))
    G = [gpu(a) for a in (*w["gate"], *w["up"])]
    note("q4 ffn q8act M=1: fused gate/up")
    out = host(qbd.gate_up_swiglu_q4_q8act(*G, xq, xd))
    g = qbd.qmm_q4_0_q8act(G[0], G[1], xq, xd)
    u = qbd.qmm_q4_0_q8act(G[2], G[3], xq, xd)
    assert np.array_equal(out.view(np.uint32), host(qbd.swiglu_f32(g, u)).view(np.uint32))
    n = w["gate"][0].shape[0]
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(35).choice(n, 512, replace=False)]))
    ref = oracle.gate_up_swiglu_q4_q8act(w["gate"][0][rows], w["gate"][1][rows], w["up"][0][rows],
                                         w["up"][1][rows], q_ref, d_ref)
    assert_swiglu("q4 ffn q8act fused gate/up M=1", out[:, rows], ref)
    note("q4 ffn q8act M=1: down")
    hq, hd = qbd.quantize_act_q8_0(gpu(h))
    hq_ref, hd_ref = oracle.quantize_act_q8_0(h)
    y = host(qbd.qmm_q4_0_q8act(gpu(w["down"][0]), gpu(w["down"][1]), hq, hd))
    _, y64, s, _ = oracle.qmm_q4_0_q8act(w["down"][0], w["down"][1], hq_ref, hd_ref)
    assert_fp32("q4 ffn q8act down M=1", y, y64, s)


# ------------------------------------- quantize + product in one call (from fp32 x)
# M = 1 over N >= 4096 with a panel of at most 4 rounds of the workgroup's
# threads takes the staged kernel that quantizes the panel in each
# workgroup (one launch: 1 to 4 rounds here, a partial last batch at K =
# 6144); the other shapes (among them K = 17408 at M = 1) run the producer
# and the product as two launches.  Either way every output byte must equal
# quantize_act_q8_0 followed by the product.
FROM_F32 = [("q8_0", 1, 4096, 32), ("q8_0", 1, 4100, 4864), ("q8_0", 1, 4864, 896), ("q8_0", 1, 151936, 896),
            ("q8_0", 1, 4100, 8192), ("q4", 1, 4100, 6144),
            ("q4", 1, 5120, 17408), ("q4", 1, 4097, 17408), ("q4", 1, 4099, 2080),
            ("gate_up_q4", 1, 17408, 5120), ("gate_up_q4", 1, 4099, 2080), ("gate_up_q4", 1, 6000, 96),
            ("q8_0", 1, 896, 4864), ("q8_0", 8, 1152, 896), ("q8_0", 32, 896, 896), ("q4", 64, 300, 1024),
            ("gate_up_q4", 8, 200, 5120), ("q8_0", 3, 0, 64),
            # two-launch shapes on the 16 x 16 tiles: persistent (4-bit fused
            # and plain, Q8_0), one tile per workgroup with 1 to 4 row groups,
            # partial last quads, 1 to 8 quads per wave
            ("gate_up_q4", 8, 8200, 5120), ("q4", 12, 8704, 2080), ("q8_0", 16, 8200, 4864),
            ("q8_0", 20, 300, 1056), ("q8_0", 45, 70, 160), ("q4", 5, 1500, 96), ("gate_up_q4", 3, 2000, 7168),
            ("q8_0", 64, 1000, 8192),
            # M=1 below the staged kernel's rows: one launch on the per-row dot4
            # kernel quantizing x in every workgroup (1 to 8 sweeps for Q8_0, to 4
            # for 4-bit, a ragged last workgroup, a partial last sweep), and one
            # sweep past that limit (two launches)
            ("q8_0", 1, 1152, 896), ("q8_0", 1, 897, 896), ("q8_0", 1, 17, 96), ("q8_0", 1, 300, 8192),
            ("q8_0", 1, 300, 8224), ("q4", 1, 1001, 8192), ("q4", 1, 33, 2080), ("gate_up_q4", 1, 1000, 4864),
            ("gate_up_q4", 1, 3, 64)]


def _from_f32_weights(rng, kind, n, k):
    q4 = kind != "q8_0"
    nmat = 2 if kind == "gate_up_q4" else 1
    if q4:
        w = [rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8) for _ in range(nmat)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03) for _ in range(nmat)]
    else:
        w = [rng.integers(-127, 128, size=(n, k), dtype=np.int8) for _ in range(nmat)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02) for _ in range(nmat)]
    return w, d


def _from_f32_call(kind, W, x, xq, xd, out):
    if kind == "q8_0":
        return qbd.qmm_q8_0_q8act_from_f32(W[0], W[1], x, xq, xd, out=out)
    if kind == "q4":
        return qbd.qmm_q4_0_q8act_from_f32(W[0], W[1], x, xq, xd, out=out)
    return qbd.gate_up_swiglu_q4_q8act_from_f32(W[0], W[1], W[2], W[3], x, xq, xd, out=out)


def _composed(kind, W, xq, xd):
    if kind == "q8_0":
        return qbd.qmm_q8_0_q8act(W[0], W[1], xq, xd)
    if kind == "q4":
        return qbd.qmm_q4_0_q8act(W[0], W[1], xq, xd)
    return qbd.gate_up_swiglu_q4_q8act(W[0], W[1], W[2], W[3], xq, xd)


@pytest.mark.parametrize("kind,m,n,k", FROM_F32)
def test_from_f32_equals_quantize_then_product(kind, m, n, k):
    import torch
    rng = np.random.default_rng(1700 + m + n + k + len(kind))
    w, d = _from_f32_weights(rng, kind, n, k)
    W = []
    for i in range(len(w)):
        W += [gpu(w[i]), gpu(d[i])]
    x_h = datagen.activations(rng, m, k, outliers=True)
    x_h[0, :32] = 0.0  # an all-zero block
    x = gpu(x_h)
    before = fingerprint(x)
    note("from_f32", kind, m, n, k)
    qbuf, xq = guarded_out((m, k), torch.int8)
    dbuf, xd = guarded_out((m, k // 32))
    ybuf, y = guarded_out((m, n))
    _from_f32_call(kind, W, x, xq, xd, y)
    first = (host(xq).copy(), host(xd).copy(), host(y).copy())
    # the producer's panel, bit for bit
    q_ref, d_ref = qbd.quantize_act_q8_0(x)
    assert np.array_equal(first[0], host(q_ref))
    assert np.array_equal(first[1].view(np.uint32), host(d_ref).view(np.uint32))
    # the product of that panel, bit for bit
    if n:
        y_ref = host(_composed(kind, W, q_ref, d_ref))
        assert np.array_equal(first[2].view(np.uint32), y_ref.view(np.uint32))
    # a second call writes the same bytes; nothing outside the outputs, and x is read only
    _from_f32_call(kind, W, x, xq, xd, y)
    assert np.array_equal(first[0], host(xq)) and np.array_equal(first[1].view(np.uint32), host(xd).view(np.uint32))
    assert np.array_equal(first[2].view(np.uint32), host(y).view(np.uint32))
    for buf, name in ((qbuf, "xq"), (dbuf, "xd"), (ybuf, "y")):
        assert_guards(buf, f"from_f32 {kind} {name}")
    assert fingerprint(x) == before
    # and against the oracle on a few rows of the smaller cases
    if kind == "q8_0" and 0 < n <= 4864 and k <= 896:
        oq, od = oracle.quantize_act_q8_0(x_h)
        assert np.array_equal(first[0], oq)
        rows = np.arange(0, n, max(1, n // 64))
        _, y64, s, _ = oracle.qmm_q8_0_q8act(w[0][rows], d[0][rows], oq, od)
        assert_fp32(f"from_f32 {kind} vs oracle", first[2][:, rows], y64, s)


@pytest.mark.parametrize("m,n", [(1, 4096), (3, 4096), (1, 50000)])
def test_from_f32_golden_ties_in_kernel(m, n):
    """The tie and reciprocal-trap blocks of the quantization golden file,
    laid end to end as one panel row, quantized inside the product launch
    (M = 1: every workgroup of the per-row kernel quantizes the row itself
    at 4096 rows, the staged kernel at 50000, past the per-row kernel's
    limit on repeated quantization) or by the producer launch ahead of the
    16 x 16 tiles (M = 3: the row three times, shifted by one block per
    row)."""
    cases = json.load(open(os.path.join(GOLDEN, "quant_ties.json")))["cases"]
    row = np.concatenate([np.array(c["x"], dtype=np.float32) for c in cases])
    x = np.stack([np.roll(row, 32 * i) for i in range(m)])
    k = x.shape[1]
    rng = np.random.default_rng(1799)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    note("from_f32 golden ties", m, n, k)
    y, q, d = qbd.qmm_q8_0_q8act_from_f32(gpu(wq), gpu(wd), gpu(x))
    for i in range(m):
        order = np.roll(np.arange(len(cases)), i)
        assert host(q)[i].reshape(len(cases), 32).tolist() == [cases[j]["q"] for j in order]
        assert [float(v) for v in host(d)[i]] == [cases[j]["d"][0] for j in order]
    _, y64, s, _ = oracle.qmm_q8_0_q8act(wq[:64], wd[:64], host(q), host(d))
    assert_fp32("from_f32 golden ties product", host(y)[:, :64], y64, s)


# ------------------------------------------- short panels staged in LDS (2..8 rows)
@pytest.mark.parametrize("q4,m,k", [(False, 2, 96), (False, 5, 8224), (False, 8, 17408), (True, 3, 7200),
                                    (True, 8, 17408), (True, 4, 8192), (True, 2, 2080)])
def test_panel_staged_kernel_equals_dot4_kernel(q4, m, k):
    """Below N = 1024 rows the dot4 kernel takes these panels (2 rows, or K
    past the reach of the 16 x 16 tiles), from 1024 on the staged one: the
    first 1023 outputs of an N = 1024 call must equal an N = 1023 call on the
    same rows bit for bit (both sum each output in the same order)."""
    wq, wd, xq, xd = q8act_inputs(2000 + m + k + q4, m, 1024, k, q4)
    W, D, XQ, XD = gpu(wq), gpu(wd), gpu(xq), gpu(xd)
    call = qbd.qmm_q4_0_q8act if q4 else qbd.qmm_q8_0_q8act
    note("panel staged vs dot4", q4, m, k)
    staged = host(call(W, D, XQ, XD))
    dot4 = host(call(W[:1023].contiguous(), D[:1023].contiguous(), XQ, XD))
    assert np.array_equal(staged[:, :1023].view(np.uint32), dot4.view(np.uint32))
    if q4:
        # the fused form too (the up matrix: the same rows reversed)
        U, UD = gpu(wq[::-1]), gpu(wd[::-1])
        f_staged = host(qbd.gate_up_swiglu_q4_q8act(W, D, U, UD, XQ, XD))
        f_dot4 = host(qbd.gate_up_swiglu_q4_q8act(W[:1023].contiguous(), D[:1023].contiguous(),
                                                  U[:1023].contiguous(), UD[:1023].contiguous(), XQ, XD))
        assert np.array_equal(f_staged[:, :1023].view(np.uint32), f_dot4.view(np.uint32))


def test_q4_down_m8_q8act_full_size_sampled():
    """The M = 8 down projection of the 4-bit FFN (5120 x 17408) on Q8
    activations (staged panel kernel), and the fused gate/up at M = 8
    (2 x 17408 x 5120, persistent 16 x 16 tiles): sampled rows against the
    oracle, among them the first and the last tile, and fused == unfused on
    every row."""
    rng = np.random.default_rng(2101)
    wq, wd = datagen.q4_weights(rng, rng, 5120, 17408)
    h = datagen.activations(rng, 8, 17408, outliers=True)
    hq, hd = oracle.quantize_act_q8_0(h)
    note("q4 down M=8 q8act full size")
    y = host(qbd.qmm_q4_0_q8act(gpu(wq), gpu(wd), gpu(hq), gpu(hd)))
    rows = np.unique(np.concatenate([np.arange(24), np.arange(5120 - 24, 5120), rng.integers(0, 5120, 48)]))
    _, y64, s, _ = oracle.qmm_q4_0_q8act(wq[rows], wd[rows], hq, hd)
    assert_fp32("q4 down M=8 q8act", y[:, rows], y64, s)
    gq, gd = datagen.q4_weights(rng, rng, 17408, 5120)
    uq, ud = datagen.q4_weights(rng, rng, 17408, 5120)
    x = datagen.activations(rng, 8, 5120, outliers=True)
    xq, xd = oracle.quantize_act_q8_0(x)
    G = [gpu(a) for a in (gq, gd, uq, ud, xq, xd)]
    note("q4 gate/up M=8 q8act full size")
    fused = host(qbd.gate_up_swiglu_q4_q8act(*G))
    unfused = host(qbd.swiglu_f32(qbd.qmm_q4_0_q8act(G[0], G[1], G[4], G[5]),
                                  qbd.qmm_q4_0_q8act(G[2], G[3], G[4], G[5])))
    assert np.array_equal(fused.view(np.uint32), unfused.view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(16), np.arange(17408 - 16, 17408), rng.integers(0, 17408, 32)]))
    ref = oracle.gate_up_swiglu_q4_q8act(gq[rows], gd[rows], uq[rows], ud[rows], xq, xd)
    assert_swiglu("q4 gate/up M=8 q8act", fused[:, rows], ref)

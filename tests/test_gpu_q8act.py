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
          (129, 70, 96), (1, 16384, 4096)]


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
@pytest.mark.parametrize("m", [1, 32, 64, 128])
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
                (1, 40001, 64), (8, 4100, 1088), (16, 4104, 1024), (2, 12300, 1024), (8, 8200, 1088)]


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
Q8_FUSED_SHAPES = [(1, 17, 96), (1, 4864, 896), (1, 4100, 4864), (2, 33, 128), (8, 130, 5120),
                   (8, 70, 5152), (5, 64, 1024), (16, 48, 2048), (1, 40001, 96), (8, 4100, 1088),
                   (13, 4112, 1024)]


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

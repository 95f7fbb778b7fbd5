"""GPU parity at activation row counts past what one grid's y dimension
holds (more than 65535 row groups of 8): the fp32-activation products then
run on the kernel that loops over row groups, and the Q8 path quantizes and
multiplies a panel of half a million rows.  Sampled rows (the first and last
eight and 40 more) are checked against the oracle."""
import numpy as np
import pytest

import block_quantized_decode_amd as qbd
from block_quantized_decode_amd import datagen
import oracle
from gpu_util import assert_fp32, assert_swiglu, gpu, host, note

pytestmark = pytest.mark.gpu

M_BIG = 65535 * 8 + 16  # 524,296 rows: 65,537 groups of 8


def sample_rows(rng, m):
    return np.unique(np.concatenate([np.arange(8), np.arange(m - 8, m), rng.choice(m, 40, replace=False)]))


@pytest.mark.parametrize("fmt", ["q8_0", "q4"])
def test_fp32_products_past_grid_rows(fmt):
    rng = np.random.default_rng(2400 + len(fmt))
    n, k = 24, 64
    x = rng.standard_normal((M_BIG, k)).astype(np.float32)
    if fmt == "q8_0":
        w = [rng.integers(-128, 128, size=(n, k), dtype=np.int8) for _ in range(2)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02) for _ in range(2)]
        plain, fused = qbd.qmv_q8_0_f32, qbd.gate_up_swiglu_q8_0
        ref_plain, ref_fused = oracle.qmv_q8_0_f32, oracle.gate_up_swiglu_q8_0
    else:
        w = [rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8) for _ in range(2)]
        d = [datagen.fp16_scales(rng, n, k // 32, 0.002, 0.03) for _ in range(2)]
        plain, fused = qbd.qmv_q4_0_f32, qbd.gate_up_swiglu_q4
        ref_plain, ref_fused = oracle.qmv_q4_0_f32, oracle.gate_up_swiglu_q4
    G = [gpu(a) for a in (w[0], d[0], w[1], d[1])]
    X = gpu(x)
    rows = sample_rows(rng, M_BIG)
    note("large-M fp32 product", fmt, M_BIG, n, k)
    y = host(plain(G[0], G[1], X))
    _, y64, s = ref_plain(w[0], d[0], x[rows])
    assert_fp32(f"{fmt} plain, M={M_BIG}", y[rows], y64, s)
    note("large-M fused gate/up", fmt, M_BIG, n, k)
    out = host(fused(*G, X))
    assert_swiglu(f"{fmt} fused, M={M_BIG}", out[rows], ref_fused(w[0], d[0], w[1], d[1], x[rows]))
    # the fused call is the unfused composition, bit for bit
    g = plain(G[0], G[1], X)
    u = plain(G[2], G[3], X)
    assert np.array_equal(out.view(np.uint32), host(qbd.swiglu_f32(g, u)).view(np.uint32))


def test_q8_path_past_grid_rows():
    rng = np.random.default_rng(2500)
    n, k = 40, 96
    x = datagen.activations(rng, M_BIG, k, outliers=True)
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = datagen.fp16_scales(rng, n, k // 32, 0.001, 0.02)
    rows = sample_rows(rng, M_BIG)
    note("large-M quantize + Q8 x Q8", M_BIG, n, k)
    xq, xd = qbd.quantize_act_q8_0(gpu(x))
    q_h, d_h = host(xq), host(xd)
    q_ref, d_ref = oracle.quantize_act_q8_0(x[rows])
    assert np.array_equal(q_h[rows], q_ref)
    assert np.array_equal(d_h[rows].view(np.uint32), d_ref.view(np.uint32))
    y = host(qbd.qmm_q8_0_q8act(gpu(wq), gpu(wd), xq, xd))
    _, y64, s, _ = oracle.qmm_q8_0_q8act(wq, wd, q_ref, d_ref)
    assert_fp32(f"qmm_q8_0_q8act, M={M_BIG}", y[rows], y64, s)

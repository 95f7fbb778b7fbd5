"""Pins of the oracle against facts outside itself.

Each pin takes the oracle module as its argument and raises AssertionError
when the oracle disagrees with: the IEEE binary16 decode of numpy's float16
type; exact rational sums (fractions.Fraction) on tiny inputs; closed forms
(one-hot activations, all-8 Q4 codes, unit scales); hand-derived rounding
cases; invariants of the quantizer; and the SiLU identities.  The pins are
called with the real oracle by test_oracle.py and with deliberately broken
copies by test_oracle_mutations.py.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np

from exact import (f16_value, f32_value, pack_q4, rat_to_f32,
                   round_half_away_exact)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE_F16 = 0x3C00  # binary16 1.0


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_q8(rng, n, k):
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = rng.uniform(0.001, 0.05, size=(n, k // 32)).astype(np.float16).view(np.uint16)
    return wq, wd


def _tiny_q4(rng, n, k):
    codes = rng.integers(0, 16, size=(n, k))
    wd = rng.uniform(0.002, 0.03, size=(n, k // 32)).astype(np.float16).view(np.uint16)
    return codes, pack_q4(codes), wd


# --------------------------------------------------------------------- fp16
def pin_fp16_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.fp16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0x0000])


def pin_fp16_named_values(orc):
    for case in _golden("fp16_values.json")["cases"]:
        got = orc.fp16_bits_to_f64(np.array([int(case["bits"], 16)], dtype=np.uint16))[0]
        want = float(Fraction(case["value"]))
        assert got == want, (case, got)


# ------------------------------------------------------------ Q8_0 x fp32
def pin_qmv_q8_exact(orc):
    """Oracle sums equal exact rational sums on tiny shapes."""
    rng = _rng(11)
    for m, n, k in [(1, 1, 32), (2, 5, 64), (3, 17, 96), (1, 4, 32)]:
        wq, wd = _tiny_q8(rng, n, k)
        x = rng.standard_normal((m, k)).astype(np.float32)
        y32, y64, s = orc.qmv_q8_0_f32(wq, wd, x)
        assert y32.shape == (m, n) and y64.shape == (m, n)
        for i in range(m):
            for j in range(n):
                exact = sum(f16_value(wd[j, kk // 32]) * int(wq[j, kk]) * f32_value(x[i, kk])
                            for kk in range(k))
                sabs = sum(abs(f16_value(wd[j, kk // 32]) * int(wq[j, kk]) * f32_value(x[i, kk]))
                           for kk in range(k))
                assert abs(Fraction(y64[i, j]) - exact) <= Fraction(2) ** -45 * sabs
                assert abs(Fraction(s[i, j]) - sabs) <= Fraction(2) ** -45 * sabs
                want32 = rat_to_f32(exact)
                ulp = float(np.spacing(np.float32(abs(want32))))
                assert abs(float(y32[i, j]) - want32) <= ulp


def pin_qmv_q8_one_hot(orc):
    """x = e_k selects exactly d[n, k/32] * q[n, k] (bitwise in fp32)."""
    rng = _rng(12)
    n, k = 9, 96
    wq, wd = _tiny_q8(rng, n, k)
    for kk in (0, 31, 32, 63, 95):
        x = np.zeros((1, k), dtype=np.float32)
        x[0, kk] = 1.0
        y32, _, _ = orc.qmv_q8_0_f32(wq, wd, x)
        for j in range(n):
            want = rat_to_f32(f16_value(wd[j, kk // 32]) * int(wq[j, kk]))
            assert float(y32[0, j]) == want


def pin_qmv_q8_unit_scale(orc):
    """d = 1 and small integer x: y is an exact integer, any order."""
    rng = _rng(13)
    m, n, k = 3, 7, 128
    wq = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    xi = rng.integers(-2, 3, size=(m, k))
    y32, y64, _ = orc.qmv_q8_0_f32(wq, wd, xi.astype(np.float32))
    want = xi.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(y64, want.astype(np.float64))
    assert np.array_equal(y32, want.astype(np.float32))


def pin_qmv_q8_scaling(orc):
    """Doubling every scale (exponent + 1) or x doubles y exactly."""
    rng = _rng(14)
    n, k = 6, 64
    wq, wd = _tiny_q8(rng, n, k)
    x = rng.standard_normal((2, k)).astype(np.float32)
    _, y, _ = orc.qmv_q8_0_f32(wq, wd, x)
    _, y2, _ = orc.qmv_q8_0_f32(wq, (wd + 0x0400).astype(np.uint16), x)
    _, y3, _ = orc.qmv_q8_0_f32(wq, wd, x * np.float32(2))
    assert np.array_equal(y2, 2 * y) and np.array_equal(y3, 2 * y)


# ---------------------------------------------------------------- Q4 x fp32
def pin_q4_layout_golden(orc):
    g = _golden("q4_block_layout.json")
    plane = np.array([g["bytes"]], dtype=np.uint8)
    codes = orc.q4_codes(plane, 32)
    assert codes.tolist() == [g["codes"]]


def pin_q4_all_eight_is_zero(orc):
    rng = _rng(21)
    n, k = 5, 96
    plane = np.full((n, k // 2), 0x88, dtype=np.uint8)
    wd = rng.uniform(0.002, 0.03, size=(n, k // 32)).astype(np.float16).view(np.uint16)
    x = rng.standard_normal((3, k)).astype(np.float32)
    y32, y64, s = orc.qmv_q4_0_f32(plane, wd, x)
    assert np.all(y64 == 0) and np.all(y32 == 0) and np.all(s == 0)


def pin_q4_one_hot(orc):
    rng = _rng(22)
    n, k = 7, 64
    codes, plane, wd = _tiny_q4(rng, n, k)
    for kk in range(0, k, 5):
        x = np.zeros((1, k), dtype=np.float32)
        x[0, kk] = 1.0
        y32, _, _ = orc.qmv_q4_0_f32(plane, wd, x)
        for j in range(n):
            want = rat_to_f32(f16_value(wd[j, kk // 32]) * (int(codes[j, kk]) - 8))
            assert float(y32[0, j]) == want


def pin_q4_exact(orc):
    rng = _rng(23)
    for m, n, k in [(1, 3, 32), (2, 5, 64), (3, 4, 96)]:
        codes, plane, wd = _tiny_q4(rng, n, k)
        x = rng.standard_normal((m, k)).astype(np.float32)
        _, y64, s = orc.qmv_q4_0_f32(plane, wd, x)
        for i in range(m):
            for j in range(n):
                terms = [f16_value(wd[j, kk // 32]) * (int(codes[j, kk]) - 8) * f32_value(x[i, kk])
                         for kk in range(k)]
                exact = sum(terms)
                sabs = sum(abs(t) for t in terms)
                assert abs(Fraction(y64[i, j]) - exact) <= Fraction(2) ** -45 * sabs
                assert abs(Fraction(s[i, j]) - sabs) <= Fraction(2) ** -45 * sabs + Fraction(0)


# ---------------------------------------------------------------- quantizer
def pin_quant_ties_golden(orc):
    g = _golden("quant_ties.json")
    for case in g["cases"]:
        x = np.array([case["x"]], dtype=np.float32)
        q, d = orc.quantize_act_q8_0(x)
        assert q.tolist() == [case["q"]], case["name"]
        assert [float(v) for v in d[0]] == [float(v) for v in case["d"]], case["name"]


def pin_quant_zero_block(orc):
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, d = orc.quantize_act_q8_0(x)
    assert np.all(q[0] == 0) and np.all(d[0] == 0)
    assert np.all(q[1, :32] == 0) and d[1, 0] == 0 and d[1, 1] > 0


def pin_quant_exact(orc):
    """d and every code equal exact-rational rounding of the stated rule."""
    rng = _rng(31)
    x = (rng.standard_normal((3, 96)) * rng.choice([1e-3, 1.0, 20.0], size=(3, 96))).astype(np.float32)
    x[2, 5] = np.float32(2.0 ** -140)          # a subnormal element
    q, d = orc.quantize_act_q8_0(x)
    for i in range(3):
        for b in range(3):
            blk = [f32_value(v) for v in x[i, 32 * b:32 * b + 32]]
            amax = max(abs(v) for v in blk)
            dd = rat_to_f32(amax / 127)
            assert float(d[i, b]) == dd
            for j, v in enumerate(blk):
                r = rat_to_f32(v / Fraction(dd)) if dd != 0 else 0.0
                assert int(q[i, 32 * b + j]) == round_half_away_exact(Fraction(r))


def pin_quant_invariants(orc):
    rng = _rng(32)
    x = rng.standard_normal((16, 320)).astype(np.float32)
    x *= np.where(rng.random(x.shape) < 0.01, 20, 1).astype(np.float32)
    q, d = orc.quantize_act_q8_0(x)
    qb = q.reshape(16, 10, 32).astype(np.int64)
    xb = x.reshape(16, 10, 32).astype(np.float64)
    assert np.all(np.max(np.abs(qb), axis=2) == 127)
    err = np.abs(xb - d[..., None].astype(np.float64) * qb)
    assert np.all(err <= d[..., None] * (0.5 + 2.0 ** -17))


def pin_quant_scale_invariance(orc):
    rng = _rng(33)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    q0, d0 = orc.quantize_act_q8_0(x)
    for j in (-20, -3, 1, 7, 30):
        q, d = orc.quantize_act_q8_0(x * np.float32(2.0 ** j))
        assert np.array_equal(q, q0)
        assert np.array_equal(d, d0 * np.float32(2.0 ** j))


# ------------------------------------------------------------ int block dots
def pin_block_dots_loops(orc):
    rng = _rng(41)
    m, n, k = 2, 3, 96
    w = rng.integers(-128, 128, size=(n, k))
    a = rng.integers(-128, 128, size=(m, k), dtype=np.int8)
    dots = orc.block_dots(w, a)
    for i in range(m):
        for j in range(n):
            for b in range(k // 32):
                want = sum(int(w[j, kk]) * int(a[i, kk]) for kk in range(32 * b, 32 * b + 32))
                assert int(dots[i, j, b]) == want


def pin_qmm_q8_exact(orc):
    rng = _rng(42)
    m, n, k = 2, 4, 96
    wq, wd = _tiny_q8(rng, n, k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    xd = rng.uniform(0.001, 0.2, size=(m, k // 32)).astype(np.float32)
    _, y64, s, dots = orc.qmm_q8_0_q8act(wq, wd, xq, xd)
    for i in range(m):
        for j in range(n):
            terms = []
            for b in range(k // 32):
                dot = sum(int(wq[j, kk]) * int(xq[i, kk]) for kk in range(32 * b, 32 * b + 32))
                assert int(dots[i, j, b]) == dot
                terms.append(f16_value(wd[j, b]) * f32_value(xd[i, b]) * dot)
            exact = sum(terms)
            sabs = sum(abs(t) for t in terms)
            assert abs(Fraction(y64[i, j]) - exact) <= Fraction(2) ** -45 * sabs


def pin_qmm_q4_exact(orc):
    rng = _rng(43)
    m, n, k = 3, 4, 64
    codes, plane, wd = _tiny_q4(rng, n, k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    xd = rng.uniform(0.001, 0.2, size=(m, k // 32)).astype(np.float32)
    _, y64, _, dots = orc.qmm_q4_0_q8act(plane, wd, xq, xd)
    for i in range(m):
        for j in range(n):
            exact = 0
            for b in range(k // 32):
                dot = sum((int(codes[j, kk]) - 8) * int(xq[i, kk]) for kk in range(32 * b, 32 * b + 32))
                assert int(dots[i, j, b]) == dot
                exact += f16_value(wd[j, b]) * f32_value(xd[i, b]) * dot
            assert abs(Fraction(y64[i, j]) - exact) <= Fraction(2) ** -45 * (abs(exact) + 1)


def pin_qmm_unit_scale_observes_dots(orc):
    """Unit weight scales and blocks with max |x| = 127 give d_x = 1, so y is
    the plain sum of the integer block dots (exact below 2^24)."""
    rng = _rng(44)
    m, n, k = 2, 5, 96
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    wd = np.full((n, k // 32), ONE_F16, dtype=np.uint16)
    xi = rng.integers(-126, 127, size=(m, k)).astype(np.float32)
    xi[:, ::32] = 127.0                                  # every block's max |x| is 127
    xq, xd = orc.quantize_act_q8_0(xi)
    assert np.all(xd == 1.0) and np.array_equal(xq.astype(np.float32), xi)
    y32, _, _, _ = orc.qmm_q8_0_q8act(wq, wd, xq, xd)
    want = xi.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(y32, want.astype(np.float32))


def pin_qmm_one_hot(orc):
    """x = 127 * 2^j * e_k quantizes to q = 127 e_k, d = 2^j, so
    y[n] = d_w[n, k/32] * 2^j * 127 * q_w[n, k]."""
    rng = _rng(45)
    n, k = 6, 64
    wq, wd = _tiny_q8(rng, n, k)
    for j, kk in [(0, 3), (-5, 40), (4, 63)]:
        x = np.zeros((1, k), dtype=np.float32)
        x[0, kk] = np.float32(127.0 * 2.0 ** j)
        xq, xd = orc.quantize_act_q8_0(x)
        y32, _, _, _ = orc.qmm_q8_0_q8act(wq, wd, xq, xd)
        for r in range(n):
            want = rat_to_f32(f16_value(wd[r, kk // 32]) * Fraction(2) ** j * 127 * int(wq[r, kk]))
            assert float(y32[0, r]) == want


# -------------------------------------------------------------------- SiLU
def pin_silu_values(orc):
    zs = [-800.0, -80.0, -20.0, -2.5, -1e-3, 0.0, 1e-3, 0.5, 2.4, 30.0, 700.0]
    got = orc.silu_f64(np.array(zs))
    for z, gz in zip(zs, got):
        want = z / (1.0 + math.exp(-z)) if -z < 700 else 0.0
        assert abs(gz - want) <= 1e-15 * abs(want) + 1e-300, (z, gz, want)
    # silu(z) - silu(-z) = z, silu(0) = 0
    z = np.linspace(-30, 30, 601)
    assert np.allclose(orc.silu_f64(z) - orc.silu_f64(-z), z, rtol=1e-13, atol=1e-13)
    assert orc.silu_f64(np.array([0.0]))[0] == 0.0


def pin_silu_lipschitz(orc):
    z = np.linspace(-40, 40, 800001)
    ds = np.abs(np.diff(orc.silu_f64(z)) / np.diff(z))
    assert ds.max() <= orc.SILU_LIPSCHITZ
    assert ds.max() > 1.09


def pin_swiglu_one_hot(orc):
    """x = e_k gives exact g = dg*(qg-8), u = du*(qu-8); out = silu(g)*u."""
    rng = _rng(51)
    n, k = 4, 64
    gcodes, gplane, gd = _tiny_q4(rng, n, k)
    ucodes, uplane, ud = _tiny_q4(rng, n, k)
    kk = 37
    x = np.zeros((1, k), dtype=np.float32)
    x[0, kk] = 1.0
    res = orc.gate_up_swiglu_q4(gplane, gd, uplane, ud, x)
    for j in range(n):
        g = float(f16_value(gd[j, 1]) * (int(gcodes[j, kk]) - 8))
        u = float(f16_value(ud[j, 1]) * (int(ucodes[j, kk]) - 8))
        assert res["g64"][0, j] == g and res["u64"][0, j] == u
        want = g / (1.0 + math.exp(-g)) * u
        assert abs(res["out64"][0, j] - want) <= 1e-15 * abs(want) + 1e-300


def pin_swiglu_fused_is_composition(orc):
    rng = _rng(52)
    n, k = 5, 96
    _, gplane, gd = _tiny_q4(rng, n, k)
    _, uplane, ud = _tiny_q4(rng, n, k)
    x = rng.standard_normal((3, k)).astype(np.float32)
    res = orc.gate_up_swiglu_q4(gplane, gd, uplane, ud, x)
    g32, _, _ = orc.qmv_q4_0_f32(gplane, gd, x)
    u32, _, _ = orc.qmv_q4_0_f32(uplane, ud, x)
    out32, _ = orc.swiglu_f32(g32, u32)
    bound = orc.swiglu_bound(res["g64"], res["u64"], res["sg"], res["su"])
    assert np.all(np.abs(out32.astype(np.float64) - res["out64"]) <= bound)


def pin_swiglu_q8_one_hot(orc):
    """Q8_0 gate/up: x = e_k gives exact g = dg*qg, u = du*qu; out = silu(g)*u."""
    rng = _rng(53)
    n, k = 4, 64
    gq, gd = _tiny_q8(rng, n, k)
    uq, ud = _tiny_q8(rng, n, k)
    kk = 45
    x = np.zeros((1, k), dtype=np.float32)
    x[0, kk] = 1.0
    res = orc.gate_up_swiglu_q8_0(gq, gd, uq, ud, x)
    for j in range(n):
        g = float(f16_value(gd[j, 1]) * int(gq[j, kk]))
        u = float(f16_value(ud[j, 1]) * int(uq[j, kk]))
        assert res["g64"][0, j] == g and res["u64"][0, j] == u
        want = g / (1.0 + math.exp(-g)) * u
        assert abs(res["out64"][0, j] - want) <= 1e-15 * abs(want) + 1e-300


def pin_swiglu_q8_fused_is_composition(orc):
    rng = _rng(54)
    n, k = 5, 96
    gq, gd = _tiny_q8(rng, n, k)
    uq, ud = _tiny_q8(rng, n, k)
    x = rng.standard_normal((3, k)).astype(np.float32)
    res = orc.gate_up_swiglu_q8_0(gq, gd, uq, ud, x)
    g32, _, _ = orc.qmv_q8_0_f32(gq, gd, x)
    u32, _, _ = orc.qmv_q8_0_f32(uq, ud, x)
    out32, _ = orc.swiglu_f32(g32, u32)
    bound = orc.swiglu_bound(res["g64"], res["u64"], res["sg"], res["su"])
    assert np.all(np.abs(out32.astype(np.float64) - res["out64"]) <= bound)


def _silu_exact_inputs(g, u):
    """silu(g) * u for exact rational g and u, through math.exp in double."""
    gf, uf = float(g), float(u)
    return gf / (1.0 + math.exp(-gf)) * uf if -gf < 700 else 0.0


def pin_swiglu_q4_q8act_one_hot(orc):
    """x = 127 * 2^j * e_k quantizes to the code 127 at k and d = 2^j in its
    block (every other block zero), so g = dg * 2^j * 127 * (qg - 8) and u
    likewise, exactly; out = silu(g) * u with SiLU on the gate side."""
    rng = _rng(55)
    n, k = 5, 96
    gcodes, gplane, gd = _tiny_q4(rng, n, k)
    ucodes, uplane, ud = _tiny_q4(rng, n, k)
    for j, kk in [(0, 7), (-6, 40), (3, 95)]:
        x = np.zeros((1, k), dtype=np.float32)
        x[0, kk] = np.float32(127.0 * 2.0 ** j)
        xq, xd = orc.quantize_act_q8_0(x)
        res = orc.gate_up_swiglu_q4_q8act(gplane, gd, uplane, ud, xq, xd)
        b = kk // 32
        for r in range(n):
            g = f16_value(gd[r, b]) * Fraction(2) ** j * 127 * (int(gcodes[r, kk]) - 8)
            u = f16_value(ud[r, b]) * Fraction(2) ** j * 127 * (int(ucodes[r, kk]) - 8)
            assert Fraction(res["g64"][0, r]) == g and Fraction(res["u64"][0, r]) == u
            want = _silu_exact_inputs(g, u)
            assert abs(res["out64"][0, r] - want) <= 1e-15 * abs(want) + 1e-300


def pin_swiglu_q4_q8act_exact(orc):
    """On tiny random inputs g and u equal the exact rational block-dot sums
    (integer dots of q - 8 against the activation codes, scaled by d_w d_x),
    and out = silu(g) * u of those exact values, gate side only."""
    rng = _rng(56)
    m, n, k = 2, 4, 64
    gcodes, gplane, gd = _tiny_q4(rng, n, k)
    ucodes, uplane, ud = _tiny_q4(rng, n, k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    xd = rng.uniform(0.001, 0.05, size=(m, k // 32)).astype(np.float32)
    res = orc.gate_up_swiglu_q4_q8act(gplane, gd, uplane, ud, xq, xd)
    for i in range(m):
        for r in range(n):
            g = u = Fraction(0)
            sg = su = Fraction(0)
            for b in range(k // 32):
                span = range(32 * b, 32 * b + 32)
                dg = sum((int(gcodes[r, kk]) - 8) * int(xq[i, kk]) for kk in span)
                du = sum((int(ucodes[r, kk]) - 8) * int(xq[i, kk]) for kk in span)
                tg = f16_value(gd[r, b]) * f32_value(xd[i, b]) * dg
                tu = f16_value(ud[r, b]) * f32_value(xd[i, b]) * du
                g += tg
                u += tu
                sg += abs(tg)
                su += abs(tu)
            assert abs(Fraction(res["g64"][i, r]) - g) <= Fraction(2) ** -45 * (sg + 1)
            assert abs(Fraction(res["u64"][i, r]) - u) <= Fraction(2) ** -45 * (su + 1)
            want = _silu_exact_inputs(g, u)
            assert abs(res["out64"][i, r] - want) <= 1e-12 * (abs(want) + 1e-12)


def pin_swiglu_q4_q8act_fused_is_composition(orc):
    """The fused Q4 x Q8-activation gate/up equals qmm_q4_0_q8act on each
    matrix followed by swiglu_f32, within the propagated bound."""
    rng = _rng(58)
    m, n, k = 3, 5, 96
    _, gplane, gd = _tiny_q4(rng, n, k)
    _, uplane, ud = _tiny_q4(rng, n, k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    xq, xd = orc.quantize_act_q8_0(x)
    res = orc.gate_up_swiglu_q4_q8act(gplane, gd, uplane, ud, xq, xd)
    g32, _, _, _ = orc.qmm_q4_0_q8act(gplane, gd, xq, xd)
    u32, _, _, _ = orc.qmm_q4_0_q8act(uplane, ud, xq, xd)
    out32, _ = orc.swiglu_f32(g32, u32)
    bound = orc.swiglu_bound(res["g64"], res["u64"], res["sg"], res["su"])
    assert np.all(np.abs(out32.astype(np.float64) - res["out64"]) <= bound)


def pin_swiglu_q4_fused_exact(orc):
    """The fp32-activation 4-bit gate/up on tiny random inputs: g and u are
    the exact rational sums, out = silu(g) * u of those."""
    rng = _rng(57)
    m, n, k = 2, 3, 64
    gcodes, gplane, gd = _tiny_q4(rng, n, k)
    ucodes, uplane, ud = _tiny_q4(rng, n, k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    res = orc.gate_up_swiglu_q4(gplane, gd, uplane, ud, x)
    for i in range(m):
        for r in range(n):
            g = sum(f16_value(gd[r, kk // 32]) * (int(gcodes[r, kk]) - 8) * f32_value(x[i, kk])
                    for kk in range(k))
            u = sum(f16_value(ud[r, kk // 32]) * (int(ucodes[r, kk]) - 8) * f32_value(x[i, kk])
                    for kk in range(k))
            assert abs(Fraction(res["g64"][i, r]) - g) <= Fraction(2) ** -40 * (abs(g) + 1)
            assert abs(Fraction(res["u64"][i, r]) - u) <= Fraction(2) ** -40 * (abs(u) + 1)
            want = _silu_exact_inputs(g, u)
            assert abs(res["out64"][i, r] - want) <= 1e-12 * (abs(want) + 1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

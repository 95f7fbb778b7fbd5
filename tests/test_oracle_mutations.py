"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin fails for each: the pins are strong enough to catch a dropped
term, a wrong sign or index, a swapped nibble order or a transposed operand.
"""
import numpy as np
import pytest

import oracle.oracle as orc
import oracle_pins


def _bad_fp16_bias(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, f / 1024.0 * 2.0 ** -14, (1 + f / 1024.0) * np.exp2(e - 16.0))
    return sign * mag


def _bad_fp16_flush_subnormals(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, 0.0, (1 + f / 1024.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _bad_q4_swapped(wq4, k):
    blocks = np.asarray(wq4, dtype=np.uint8).reshape(len(wq4), k // 32, 16).astype(np.int64)
    return np.concatenate([blocks >> 4, blocks & 15], axis=2).reshape(len(wq4), k)


def _bad_q4_interleaved(wq4, k):
    blocks = np.asarray(wq4, dtype=np.uint8).reshape(len(wq4), k // 32, 16).astype(np.int64)
    return np.stack([blocks & 15, blocks >> 4], axis=3).reshape(len(wq4), k)


def _bad_dequant_q4_no_offset(wq4, wd, k):
    codes = orc.q4_codes(wq4, k)
    d = orc.fp16_bits_to_f64(wd).reshape(codes.shape[0], k // 32)
    return np.repeat(d, 32, axis=1) * codes


def _bad_dequant_q4_scale_shifted(wq4, wd, k):
    codes = orc.q4_codes(wq4, k)
    d = orc.fp16_bits_to_f64(wd).reshape(codes.shape[0], k // 32)
    return np.repeat(np.roll(d, 1, axis=1), 32, axis=1) * (codes - 8).astype(np.float64)


def _bad_dequant_q8_tiled(wq, wd):
    n, k = wq.shape
    d = orc.fp16_bits_to_f64(wd).reshape(n, k // 32)
    return np.tile(d, (1, 32)) * wq.astype(np.float64)


def _bad_round_even(r):
    return np.round(np.asarray(r, dtype=np.float64))


def _bad_round_floor(r):
    return np.floor(np.asarray(r, dtype=np.float64) + 0.5)


def _bad_quant_128(x):
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    xb = x.reshape(m, k // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(128.0)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d)
    q = orc.round_half_away((xb / safe[..., None]).astype(np.float32))
    return np.clip(q, -127, 127).astype(np.int8).reshape(m, k), d


def _bad_quant_reciprocal(x):
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    xb = x.reshape(m, k // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    inv = np.where(d == 0, np.float32(0), np.float32(1) / np.where(d == 0, np.float32(1), d))
    q = orc.round_half_away((xb * inv[..., None].astype(np.float32)).astype(np.float32))
    return np.clip(q, -127, 127).astype(np.int8).reshape(m, k), d


def _bad_block_dots_dropped(wcodes, xq):
    w = np.asarray(wcodes).astype(np.int64)
    a = np.asarray(xq).astype(np.int64)
    n, k = w.shape
    wb = w.reshape(n, k // 32, 32)[:, :, :31]
    ab = a.reshape(a.shape[0], k // 32, 32)[:, :, :31]
    return np.einsum("mbi,nbi->mnb", ab, wb)


def _bad_block_dots_int16(wcodes, xq):
    w = np.asarray(wcodes).astype(np.int16)
    a = np.asarray(xq).astype(np.int16)
    n, k = w.shape
    wb = w.reshape(n, k // 32, 32)
    ab = a.reshape(a.shape[0], k // 32, 32)
    # products and sums wrap around in 16 bits
    return np.einsum("mbi,nbi->mnb", ab, wb, dtype=np.int16).astype(np.int64)


def _bad_scaled_sum_no_dx(dots, dw, dx):
    t = dw[None, :, :] * dots.astype(np.float64)
    return t.sum(axis=2), np.abs(t).sum(axis=2)


def _bad_matvec_transposed(w, x):
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    wt = w.reshape(w.shape[1], w.shape[0]) if w.shape[0] != w.shape[1] else w.T
    y = x64 @ wt if x64.shape[1] == wt.shape[0] else x64 @ wt.T
    return y, np.abs(x64) @ np.abs(wt if x64.shape[1] == wt.shape[0] else wt.T)


def _bad_silu_sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _bad_silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


_GATE_UP_Q4 = orc.gate_up_swiglu_q4
_GATE_UP_Q8 = orc.gate_up_swiglu_q8_0


def _bad_gate_up_q4_swapped(gq, gd, uq, ud, x):
    return _GATE_UP_Q4(uq, ud, gq, gd, x)  # silu applied to the up projection


def _bad_gate_up_q8_swapped(gq, gd, uq, ud, x):
    return _GATE_UP_Q8(uq, ud, gq, gd, x)


def _bad_gate_up_q8_gate_twice(gq, gd, uq, ud, x):
    return _GATE_UP_Q8(gq, gd, gq, gd, x)  # the up weights never read


def _bad_gate_up_q4_gate_twice(gq, gd, uq, ud, x):
    return _GATE_UP_Q4(gq, gd, gq, gd, x)


_GATE_UP_Q4_Q8ACT = orc.gate_up_swiglu_q4_q8act


def _bad_gate_up_q4_q8act_swapped(gq, gd, uq, ud, xq, xd):
    return _GATE_UP_Q4_Q8ACT(uq, ud, gq, gd, xq, xd)


def _bad_gate_up_q4_q8act_gate_twice(gq, gd, uq, ud, xq, xd):
    return _GATE_UP_Q4_Q8ACT(gq, gd, gq, gd, xq, xd)


def _bad_gate_up_q4_q8act_sigmoid(gq, gd, uq, ud, xq, xd):
    res = _GATE_UP_Q4_Q8ACT(gq, gd, uq, ud, xq, xd)
    g, u = res["g64"], res["u64"]
    with np.errstate(over="ignore"):
        res["out64"] = u / (1.0 + np.exp(-g))  # sigmoid(g) * u
    res["out32"] = res["out64"].astype(np.float32)
    return res


MUTANTS = {
    "fp16 exponent bias 16": ("fp16_bits_to_f64", _bad_fp16_bias),
    "fp16 subnormals flushed to zero": ("fp16_bits_to_f64", _bad_fp16_flush_subnormals),
    "Q4 nibble halves swapped": ("q4_codes", _bad_q4_swapped),
    "Q4 nibbles interleaved": ("q4_codes", _bad_q4_interleaved),
    "Q4 offset 8 dropped": ("dequant_q4", _bad_dequant_q4_no_offset),
    "Q8 scale index k%B": ("dequant_q8_0", _bad_dequant_q8_tiled),
    "Q4 scale of the previous block": ("dequant_q4", _bad_dequant_q4_scale_shifted),
    "round half to even": ("round_half_away", _bad_round_even),
    "round as floor(r+0.5)": ("round_half_away", _bad_round_floor),
    "quantize divides by 128": ("quantize_act_q8_0", _bad_quant_128),
    "quantize by reciprocal": ("quantize_act_q8_0", _bad_quant_reciprocal),
    "block dot drops a term": ("block_dots", _bad_block_dots_dropped),
    "block dot in 16-bit integers": ("block_dots", _bad_block_dots_int16),
    "activation scale dropped": ("_scaled_sum", _bad_scaled_sum_no_dx),
    "weights transposed": ("_matvec_f64", _bad_matvec_transposed),
    "silu is sigmoid": ("silu_f64", _bad_silu_sigmoid),
    "silu sign flipped": ("silu_f64", _bad_silu_sign),
    "Q4 gate/up: silu on the up side": ("gate_up_swiglu_q4", _bad_gate_up_q4_swapped),
    "Q8_0 gate/up: silu on the up side": ("gate_up_swiglu_q8_0", _bad_gate_up_q8_swapped),
    "Q8_0 gate/up: gate weights for both": ("gate_up_swiglu_q8_0", _bad_gate_up_q8_gate_twice),
    "Q4 gate/up: gate weights for both": ("gate_up_swiglu_q4", _bad_gate_up_q4_gate_twice),
    "Q4 x Q8 gate/up: silu on the up side": ("gate_up_swiglu_q4_q8act", _bad_gate_up_q4_q8act_swapped),
    "Q4 x Q8 gate/up: gate weights for both": ("gate_up_swiglu_q4_q8act", _bad_gate_up_q4_q8act_gate_twice),
    "Q4 x Q8 gate/up: sigmoid instead of silu": ("gate_up_swiglu_q4_q8act", _bad_gate_up_q4_q8act_sigmoid),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(orc, attr, bad)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception:  # an assertion or a shape error both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"

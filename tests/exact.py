"""Exact rational arithmetic used to pin the oracle (pure Python, tiny inputs).

Nothing here is shared with the oracle or the HIP library: binary16 values
are decoded through numpy's own float16 type, sums are formed with
fractions.Fraction, and fp32 rounding is an integer round-to-nearest-even of
the exact rational.
"""

from fractions import Fraction

import numpy as np


def f16_value(bits):
    """Exact value of a binary16 pattern, decoded by numpy's float16."""
    v = np.array([bits], dtype=np.uint16).view(np.float16)[0]
    return Fraction(float(v))


def f32_value(x):
    return Fraction(float(np.float32(x)))


def rat_to_f32(q):
    """Round a rational to the nearest binary32 value, ties to even."""
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                   # below 2^-126 the quantum is fixed
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    whole = n.numerator // n.denominator
    rem = n - whole
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    val = sign * float(whole * quantum)
    if abs(val) > float(np.finfo(np.float32).max):
        return sign * float("inf")
    return val


def round_half_away_exact(q):
    """Nearest integer to a rational, ties away from zero."""
    q = Fraction(q)
    a = abs(q)
    n = (a + Fraction(1, 2)).__floor__()
    return int(n) if q >= 0 else -int(n)


def pack_q4(codes):
    """Pack codes int [N][K] (0..15) into the Q4 plane uint8 [N][K/2].

    Block b of a row occupies bytes 16b..16b+15; byte j of the block holds
    code 32b+j in bits 0-3 and code 32b+16+j in bits 4-7.
    """
    codes = np.asarray(codes)
    n, k = codes.shape
    out = np.zeros((n, k // 2), dtype=np.uint8)
    for r in range(n):
        for b in range(k // 32):
            for j in range(16):
                lo = int(codes[r, 32 * b + j])
                hi = int(codes[r, 32 * b + 16 + j])
                out[r, 16 * b + j] = lo | (hi << 4)
    return out

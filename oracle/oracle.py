"""Reference oracle for block-quantized decode matmuls.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, table or helper with the HIP
library; the two meet only in the seeded input generators, which hold none of
the arithmetic below.

Every function is the plain definition of the operation, written out with
numpy in float64 (floating point) or int64 (integer codes and dots).  No
blocking, fusion or reordering beyond what the definition states; a library
matmul serves as the summation step where noted.  Functions that return
floating results also return S = sum |terms| per output, which the parity
tolerance |y_gpu - y_ref| <= 1e-4 * S + 1e-6 is stated in.

Formats (sources cited per function):
  Q8_0 block : 32 signed 8-bit codes q and one IEEE binary16 scale d; the
               weight is d*q.  Stored as two planes: codes int8 [N][K]
               (row n = output n, K contiguous) and scales uint16 [N][K/32]
               holding binary16 bit patterns.
  Q4 block   : 32 four-bit codes q in 0..15 and one binary16 scale d; the
               weight is d*(q-8).  Codes plane uint8 [N][K/2]: block b of a
               row is bytes [16b, 16b+16); byte j carries code 32b+j in its low
               nibble and code 32b+16+j in its high nibble.
  Q8 activation block : 32 int8 codes and one fp32 scale, d = max|x|/127,
               q = round-half-away(x/d) (fp32 division), d = 0 and q = 0 for
               an all-zero block.
"""

import numpy as np

QK = 32  # codes per block, for every format here


# ---------------------------------------------------------------------------
# binary16 decode (IEEE 754-2008 binary16: 1 sign, 5 exponent, 10 fraction bits)
# ---------------------------------------------------------------------------
def fp16_bits_to_f64(bits):
    """Decode binary16 bit patterns to float64, from the IEEE definition.

    The per-block scale of both weight formats is an fp16 value ("broadcasts
    the per-block fp16 scale d": Lumen v0.2.0 release page, section
    "Phase 7.D - Q8-native fused matmul").  Normal: (1 + f/1024) * 2^(e-15);
    subnormal (e == 0): f/1024 * 2^-14; e == 31: inf (f == 0) or NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    subnormal = (f / 1024.0) * 2.0 ** -14
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _check_k(k):
    if k <= 0 or k % QK != 0:
        raise ValueError(f"K must be a positive multiple of {QK}, got {k}")


# ---------------------------------------------------------------------------
# weight decode
# ---------------------------------------------------------------------------
def dequant_q8_0(wq, wd):
    """Q8_0 weights as float64: w[n,k] = d[n, k//32] * q[n,k] (exact in fp64).

    Native Q8_0 blocks kept end to end, one fp16 scale per 32 codes, one
    output row per weight row with K contiguous (Lumen v0.2.0 release page,
    "Phase 7.D - Q8-native fused matmul").
    """
    wq = np.asarray(wq)
    n, k = wq.shape
    _check_k(k)
    d = fp16_bits_to_f64(wd).reshape(n, k // QK)
    return np.repeat(d, QK, axis=1) * wq.astype(np.float64)


def q4_codes(wq4, k):
    """Unpack the Q4 codes plane uint8 [N][K/2] to codes int64 [N][K] in 0..15.

    Within block b, byte j holds code 32b+j (low nibble) and 32b+16+j (high
    nibble).  The pages name the 4-bit format ("Q4 gate/up": LSE v0.4.16
    release page, "Combined M8 Q4 gate/up execution") without its byte order;
    this order is the reading adopted here.
    """
    wq4 = np.asarray(wq4, dtype=np.uint8)
    _check_k(k)
    n = wq4.shape[0]
    if wq4.shape != (n, k // 2):
        raise ValueError("Q4 codes plane must be [N][K/2]")
    blocks = wq4.reshape(n, k // QK, QK // 2).astype(np.int64)
    low = blocks & 0x0F          # codes 0..15 of the block
    high = (blocks >> 4) & 0x0F  # codes 16..31 of the block
    return np.concatenate([low, high], axis=2).reshape(n, k)


def dequant_q4(wq4, wd, k):
    """Q4 weights as float64: w[n,k] = d[n, k//32] * (q[n,k] - 8) (exact)."""
    codes = q4_codes(wq4, k)
    n = codes.shape[0]
    d = fp16_bits_to_f64(wd).reshape(n, k // QK)
    return np.repeat(d, QK, axis=1) * (codes - 8).astype(np.float64)


# ---------------------------------------------------------------------------
# weight x fp32-activation products
# ---------------------------------------------------------------------------
def _matvec_f64(w, x):
    """y[m,n] = sum_k x[m,k] * w[n,k] in float64; S[m,n] = sum_k |x*w|.

    Each term is exact in float64 (fp16 scale 11 bits x code <= 8 bits x fp32
    activation 24 bits <= 43 bits); the library matmul only sums them.
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x64)):
        raise ValueError("activations must be finite")
    y = x64 @ w.T
    s = np.abs(x64) @ np.abs(w).T
    return y, s


def qmv_q8_0_f32(wq, wd, x):
    """y = x . W^T for Q8_0 weights and fp32 activations x [M][K].

    Q8-native fused matmul with no dequantized weight copy (Lumen v0.2.0
    release page, "Phase 7.D - Q8-native fused matmul"); per-row decode GEMV
    at M = 1 ("Phase 7.C - 1xN 4-accumulator decode kernel", same page).
    Returns (y as float32, y as float64, S).
    """
    w = dequant_q8_0(wq, wd)
    y, s = _matvec_f64(w, x)
    return y.astype(np.float32), y, s


def qmv_q4_0_f32(wq4, wd, x):
    """y = x . W^T for Q4 weights (d*(q-8)) and fp32 activations x [M][K].

    One projection of the gate/up pair (LSE v0.4.16 release page, "Combined
    M8 Q4 gate/up execution": each projection accumulated on its own).
    Returns (y as float32, y as float64, S).
    """
    x = np.asarray(x, dtype=np.float32)
    w = dequant_q4(wq4, wd, x.shape[1])
    y, s = _matvec_f64(w, x)
    return y.astype(np.float32), y, s


# ---------------------------------------------------------------------------
# SwiGLU
# ---------------------------------------------------------------------------
def silu_f64(z):
    """silu(z) = z / (1 + exp(-z)) in float64.

    The pages use an "existing SiLU intrinsic" without defining it (LSE
    v0.4.16 release page, "Combined M8 Q4 gate/up execution"); this is the
    standard definition, applied to the gate projection only.
    """
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        e = np.exp(-z)
    return z / (1.0 + e)


def swiglu_f32(g, u):
    """out = silu(g) * u for fp32 g and u, evaluated in float64.

    Returns (out as float32, out as float64).
    """
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    u64 = np.asarray(u, dtype=np.float32).astype(np.float64)
    out = silu_f64(g64) * u64
    return out.astype(np.float32), out


def gate_up_swiglu_q4(gq, gd, uq, ud, x):
    """out = silu(x . Wg^T) * (x . Wu^T), Q4 gate and up weights, fp32 x.

    The combined gate/up SwiGLU consumer: one shared activation panel, two
    independently accumulated projections, SiLU on the gate, no gate
    temporary (LSE v0.4.16 release page, "Combined M8 Q4 gate/up execution").
    Returns a dict with out32, out64 and the projections g64, u64 with their
    term sums sg, su (for the error bound of the product).
    """
    _, g64, sg = qmv_q4_0_f32(gq, gd, x)
    _, u64, su = qmv_q4_0_f32(uq, ud, x)
    out64 = silu_f64(g64) * u64
    return {"out32": out64.astype(np.float32), "out64": out64,
            "g64": g64, "u64": u64, "sg": sg, "su": su}


def gate_up_swiglu_q8_0(gq, gd, uq, ud, x):
    """out = silu(x . Wg^T) * (x . Wu^T) with Q8_0 gate and up weights, fp32 x.

    The same combined gate/up SwiGLU consumer (LSE v0.4.16 release page,
    "Combined M8 Q4 gate/up execution") on the 8-bit blocks of the decode
    layer's gate and up projections.  Returns a dict like gate_up_swiglu_q4.
    """
    _, g64, sg = qmv_q8_0_f32(gq, gd, x)
    _, u64, su = qmv_q8_0_f32(uq, ud, x)
    out64 = silu_f64(g64) * u64
    return {"out32": out64.astype(np.float32), "out64": out64,
            "g64": g64, "u64": u64, "sg": sg, "su": su}


# ---------------------------------------------------------------------------
# activation quantization
# ---------------------------------------------------------------------------
def round_half_away(r):
    """Round to nearest, ties away from zero, exactly (float64 arithmetic).

    r is an fp32 value with |r| <= 127.5, so r +/- 0.5 is exact in float64.
    """
    r = np.asarray(r, dtype=np.float64)
    return np.where(r >= 0.0, np.floor(r + 0.5), -np.floor(-r + 0.5))


def quantize_act_q8_0(x):
    """Per-32-block Q8 activation quantization of fp32 x [M][K].

    The activation quantization that feeds the Q8 x Q8 matmul (Lumen v0.4.0
    release page, "Phase 7.M - Q8xQ8 AVX2 int dot": "activation quantization
    pipeline"); also the activation panel producer of LSE v0.4.15 release
    page, "Changes".  Rule adopted here, per row m and block b:
      a = max |x| over the block (exact),
      d = fl32(a / 127)          correctly rounded fp32 division,
      q = round-half-away(fl32(x / d)), clamped to [-127, 127];
      a == 0  ->  d = 0 and every q = 0.
    Returns (codes int8 [M][K], scales float32 [M][K/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    _check_k(k)
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    xb = x.reshape(m, k // QK, QK)
    amax = np.max(np.abs(xb), axis=2)                      # float32, exact
    d = (amax / np.float32(127.0)).astype(np.float32)      # fp32 division
    safe = np.where(d == 0, np.float32(1.0), d)
    r = (xb / safe[..., None]).astype(np.float32)          # fp32 division
    q = round_half_away(r)
    q = np.where(d[..., None] == 0, 0.0, q)
    q = np.clip(q, -127, 127)
    return q.astype(np.int8).reshape(m, k), d


# ---------------------------------------------------------------------------
# weight x Q8-activation products (exact int32 block dots)
# ---------------------------------------------------------------------------
def block_dots(wcodes, xq):
    """dot[m,n,b] = sum_{i<32} wcodes[n,32b+i] * xq[m,32b+i], exact int64.

    wcodes: int [N][K] signed weight codes (q for Q8_0, q-8 for Q4);
    xq: int8 [M][K] activation codes.  The exact integer block dot of the
    Q8 x Q8 kernel (Lumen v0.4.0 release page, "Phase 7.M - Q8xQ8 AVX2 int
    dot"; one fp32 sub-accumulator per block, "Phase 7.O - 4-accumulator
    VNNI kernel").
    """
    w = np.asarray(wcodes).astype(np.int64)
    a = np.asarray(xq).astype(np.int64)
    n, k = w.shape
    m = a.shape[0]
    _check_k(k)
    wb = w.reshape(n, k // QK, QK)
    ab = a.reshape(m, k // QK, QK)
    return np.einsum("mbi,nbi->mnb", ab, wb)


def _scaled_sum(dots, dw, dx):
    """y[m,n] = sum_b dw[n,b] * dx[m,b] * dot[m,n,b] in float64, and S."""
    t = dx.astype(np.float64)[:, None, :] * dw[None, :, :] * dots.astype(np.float64)
    return t.sum(axis=2), np.abs(t).sum(axis=2)


def qmm_q8_0_q8act(wq, wd, xq, xd):
    """y = sum_b d_w * d_x * dot_b, Q8_0 weights x Q8 activations.

    Per-block exact int dot then fp32-scale accumulation (Lumen v0.4.0
    release page, "Phase 7.M" and "Phase 7.O"); at M = 32 this is the pp32
    prefill shape (Lumen v0.5.0 release page, "Headline").
    Returns (y float32, y float64, S, dots int64 [M][N][K/32]).
    """
    wq = np.asarray(wq)
    n, k = wq.shape
    dw = fp16_bits_to_f64(wd).reshape(n, k // QK)
    dots = block_dots(wq, xq)
    y, s = _scaled_sum(dots, dw, np.asarray(xd, dtype=np.float32))
    return y.astype(np.float32), y, s, dots


def qmm_q4_0_q8act(wq4, wd, xq, xd):
    """y = sum_b d_w * d_x * dot_b with dot = sum (q_w - 8) * q_x, Q4 weights.

    The prefill-sized product (LSE v0.4.16 release page, "Retained
    optimizations and compatibility": M1024 prefill panels).
    Returns (y float32, y float64, S, dots int64 [M][N][K/32]).
    """
    xq = np.asarray(xq)
    k = xq.shape[1]
    codes = q4_codes(wq4, k) - 8
    n = codes.shape[0]
    dw = fp16_bits_to_f64(wd).reshape(n, k // QK)
    dots = block_dots(codes, xq)
    y, s = _scaled_sum(dots, dw, np.asarray(xd, dtype=np.float32))
    return y.astype(np.float32), y, s, dots


def gate_up_swiglu_q4_q8act(gq, gd, uq, ud, xq, xd):
    """out = silu(g) * u with g, u the Q4 x Q8-activation products.

    The combined gate/up consumer (LSE v0.4.16 release page, "Combined M8 Q4
    gate/up execution": both projections accumulated on their own, SiLU on
    the gate) fed by the per-block Q8 activation panel of the prefill
    product (same page, "Retained optimizations and compatibility").
    Returns a dict like gate_up_swiglu_q4.
    """
    _, g64, sg, _ = qmm_q4_0_q8act(gq, gd, xq, xd)
    _, u64, su, _ = qmm_q4_0_q8act(uq, ud, xq, xd)
    out64 = silu_f64(g64) * u64
    return {"out32": out64.astype(np.float32), "out64": out64,
            "g64": g64, "u64": u64, "sg": sg, "su": su}


# ---------------------------------------------------------------------------
# tolerances
# ---------------------------------------------------------------------------
def fp32_bound(s):
    """Allowed |y_gpu - y_ref| for an fp32 output with term sum S."""
    return 1e-4 * np.asarray(s, dtype=np.float64) + 1e-6


SILU_LIPSCHITZ = 1.1   # max |silu'(z)| is about 1.0998, near z = 2.4
EVAL_REL = 2.0 ** -18  # device exp, division and product, relative


def swiglu_bound(g64, u64, sg, su):
    """Allowed |out_gpu - out_ref| when g and u carry fp32-product errors.

    With |g~ - g| <= Eg and |u~ - u| <= Eu (Eg, Eu from fp32_bound):
      |silu(g~) u~ - silu(g) u| <= 1.1 Eg (|u| + Eu) + |silu(g)| Eu,
    plus the relative error of evaluating silu and the product in fp32.
    """
    eg = fp32_bound(sg)
    eu = fp32_bound(su)
    prop = SILU_LIPSCHITZ * eg * (np.abs(u64) + eu) + np.abs(silu_f64(g64)) * eu
    out = np.abs(silu_f64(g64) * u64)
    return prop * (1.0 + EVAL_REL) + EVAL_REL * out + 1e-6


def swiglu_elementwise_bound(out64):
    """Allowed |out_gpu - out_ref| for swiglu_f32 on exact fp32 inputs."""
    return EVAL_REL * np.abs(np.asarray(out64, dtype=np.float64)) + 1e-30

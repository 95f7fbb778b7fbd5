"""Seeded synthetic inputs for the block-quantized decode matmuls.

This module draws random numbers and nothing else: it holds none of the
arithmetic of the matmuls, the quantizer or the SwiGLU.  Both the HIP path
and the reference oracle consume what it returns.

Recipe (per workload index c):
  * numpy Generator streams spawned from SeedSequence(1234 + c);
  * Q8_0 codes: integers uniform on [-127, 127] (int8);
  * Q4 codes plane: bytes uniform on [0, 255]; each nibble of a uniform byte
    is independently uniform on 0..15, so the 4-bit codes are uniform;
  * fp16 scales: float64 uniform on [lo, hi], rounded to nearest binary16 and
    returned as uint16 bit patterns;
  * activations: float64 standard normal cast to float32, optionally with
    each element independently multiplied by 20 with probability 0.01.

Workload shapes (M activation rows, N output features, K input features):
  * single GEMV          M=1,    N=896,    K=896
  * decode layer (Qwen2.5-0.5B-shaped, Q8_0): qkv 896->1152, wo 896->896,
    gate and up 896->4864, down 4864->896, lm_head 896->151936; M=1
  * Q8 x Q8: the decode-layer shapes at M=1 and M=32 (pp32)
  * fused gate/up SwiGLU: M=8,    N=17408, K=5120, Q4 weights
  * prefill:              M=1024, N=17408, K=5120, Q4 weights, Q8 activations
"""

import numpy as np

SEED_BASE = 1234

# (name, N, K) of one Qwen2.5-0.5B-shaped decode layer, then the LM head.
DECODE_LAYER = (
    ("qkv", 1152, 896),
    ("wo", 896, 896),
    ("gate", 4864, 896),
    ("up", 4864, 896),
    ("down", 896, 4864),
)
LM_HEAD = ("lm_head", 151936, 896)

Q8_SCALE_RANGE = (0.001, 0.02)
Q4_SCALE_RANGE = (0.002, 0.03)

SINGLE_GEMV = dict(M=1, N=896, K=896)
GATE_UP = dict(M=8, N=17408, K=5120)
# 4-bit FFN of the 27B-class target (gate/up 5120 -> 17408, down 17408 -> 5120)
Q4_FFN = (("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408))
DOWN_M8 = dict(M=8, N=5120, K=17408)
PREFILL = dict(M=1024, N=17408, K=5120)
PP32_M = 32
OUTLIER_PROB = 0.01
OUTLIER_GAIN = 20.0


def streams(workload_index, count):
    """`count` independent generators for workload `workload_index`."""
    ss = np.random.SeedSequence(SEED_BASE + int(workload_index))
    return [np.random.default_rng(s) for s in ss.spawn(count)]


def q8_codes(rng, n, k):
    """int8 [n][k], uniform on [-127, 127]."""
    return rng.integers(-127, 128, size=(n, k), dtype=np.int8)


def q4_code_bytes(rng, n, k):
    """uint8 [n][k/2]; every nibble uniform on 0..15."""
    return rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def fp16_scales(rng, n, nblocks, lo, hi):
    """uint16 [n][nblocks] binary16 bit patterns of uniform draws on [lo, hi]."""
    v = rng.uniform(lo, hi, size=(n, nblocks))
    return v.astype(np.float16).view(np.uint16)


def activations(rng, m, k, outliers=False):
    """float32 [m][k] standard normal, optionally with 1% x20 outliers."""
    x = rng.standard_normal(size=(m, k))
    if outliers:
        hit = rng.random(size=(m, k)) < OUTLIER_PROB
        x = np.where(hit, x * OUTLIER_GAIN, x)
    return x.astype(np.float32)


def q8_weights(rng_codes, rng_scales, n, k):
    """(codes int8 [n][k], scales uint16 [n][k/32]) of a Q8_0 matrix."""
    return (q8_codes(rng_codes, n, k),
            fp16_scales(rng_scales, n, k // 32, *Q8_SCALE_RANGE))


def q4_weights(rng_codes, rng_scales, n, k):
    """(codes uint8 [n][k/2], scales uint16 [n][k/32]) of a Q4 matrix."""
    return (q4_code_bytes(rng_codes, n, k),
            fp16_scales(rng_scales, n, k // 32, *Q4_SCALE_RANGE))


def single_gemv(n=SINGLE_GEMV["N"], k=SINGLE_GEMV["K"], m=SINGLE_GEMV["M"]):
    """Inputs of the single Q8_0 GEMV workload (index 0)."""
    rc, rs, rx = streams(0, 3)
    wq, wd = q8_weights(rc, rs, n, k)
    return wq, wd, activations(rx, m, k)


def _keyed(workload_index, key, count):
    """`count` generators of a keyed sub-sequence of workload `workload_index`."""
    ss = np.random.SeedSequence(SEED_BASE + int(workload_index), spawn_key=(int(key),))
    return [np.random.default_rng(s) for s in ss.spawn(count)]


def decode_layer_weights(layer_index=0):
    """Q8_0 weights of decode layer copy `layer_index` (index 1).

    Returns dict name -> (codes int8 [N][K], scales uint16 [N][K/32]).
    """
    r = _keyed(1, 1000 + int(layer_index), 2 * len(DECODE_LAYER))
    return {name: q8_weights(r[2 * i], r[2 * i + 1], n, k)
            for i, (name, n, k) in enumerate(DECODE_LAYER)}


def lm_head_weights(copy_index=0):
    """Q8_0 LM-head weights, copy `copy_index` (index 1)."""
    rc, rs = _keyed(1, 2000 + int(copy_index), 2)
    _, n, k = LM_HEAD
    return q8_weights(rc, rs, n, k)


def decode_activations(m=1):
    """fp32 activations for the two decode input widths: {896: x, 4864: x}."""
    r896, r4864 = _keyed(1, 3000 + int(m), 2)
    return {896: activations(r896, m, 896), 4864: activations(r4864, m, 4864)}


def q8q8_inputs(n, k, m):
    """Q8_0 weights and outlier-bearing activations for the Q8 x Q8 path."""
    rc, rs, rx = streams(2, 3)
    wq, wd = q8_weights(rc, rs, n, k)
    return wq, wd, activations(rx, m, k, outliers=True)


def gate_up_inputs(n=GATE_UP["N"], k=GATE_UP["K"], m=GATE_UP["M"]):
    """Q4 gate and up weights and fp32 activations (index 3)."""
    r = streams(3, 5)
    gq, gd = q4_weights(r[0], r[1], n, k)
    uq, ud = q4_weights(r[2], r[3], n, k)
    return gq, gd, uq, ud, activations(r[4], m, k)


def prefill_inputs(n=PREFILL["N"], k=PREFILL["K"], m=PREFILL["M"]):
    """Q4 gate and up weights and fp32 activations to quantize (index 4)."""
    r = streams(4, 5)
    gq, gd = q4_weights(r[0], r[1], n, k)
    uq, ud = q4_weights(r[2], r[3], n, k)
    return gq, gd, uq, ud, activations(r[4], m, k)


def q4_ffn_weights(copy_index=0):
    """4-bit FFN weights (gate, up, down) of copy `copy_index` (index 5).

    Returns dict name -> (codes uint8 [N][K/2], scales uint16 [N][K/32]).
    """
    r = _keyed(5, 1000 + int(copy_index), 2 * len(Q4_FFN))
    return {name: q4_weights(r[2 * i], r[2 * i + 1], n, k) for i, (name, n, k) in enumerate(Q4_FFN)}


def q4_ffn_activations(m=1):
    """fp32 activations of the FFN input (K = 5120) and of the down
    projection's input (K = 17408) at M = m (index 5)."""
    ra, rb = _keyed(5, 3000 + int(m), 2)
    return activations(ra, m, Q4_FFN[0][2]), activations(rb, m, Q4_FFN[2][2])

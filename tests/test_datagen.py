"""The seeded input generators against the recipe they state: ranges,
rounding of the fp16 scales, the outlier rule, the workload shapes, and
determinism (same index, same bytes; another copy index, other bytes)."""
import numpy as np

from block_quantized_decode_amd import datagen


def test_q8_codes_range_and_spread():
    (rng,) = datagen.streams(90, 1)
    q = datagen.q8_codes(rng, 256, 1024)
    assert q.dtype == np.int8 and q.shape == (256, 1024)
    assert q.min() == -127 and q.max() == 127  # -128 is never drawn
    counts = np.bincount(q.astype(np.int64).ravel() + 127, minlength=255)
    assert counts.min() > 0.7 * counts.mean()  # roughly uniform over all 255 values


def test_q4_nibbles_uniform():
    (rng,) = datagen.streams(91, 1)
    b = datagen.q4_code_bytes(rng, 512, 1024)
    assert b.dtype == np.uint8 and b.shape == (512, 512)
    for nib in (b & 15, b >> 4):
        counts = np.bincount(nib.ravel(), minlength=16)
        assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()


def test_fp16_scales_are_rounded_uniform_draws():
    (rng,) = datagen.streams(92, 1)
    lo, hi = datagen.Q4_SCALE_RANGE
    bits = datagen.fp16_scales(rng, 300, 160, lo, hi)
    assert bits.dtype == np.uint16
    v = bits.view(np.float16).astype(np.float64)
    assert v.min() >= np.float16(lo) and v.max() <= np.float16(hi)
    # each value is the nearest binary16 of a draw from the same stream
    (rng2,) = datagen.streams(92, 1)
    raw = rng2.uniform(lo, hi, size=(300, 160))
    assert np.array_equal(bits, raw.astype(np.float16).view(np.uint16))
    assert np.all(np.abs(v - raw) <= np.spacing(np.float16(hi)).astype(np.float64) / 2)


def test_activations_normal_with_outliers():
    (rng,) = datagen.streams(93, 1)
    x = datagen.activations(rng, 64, 4096)
    assert x.dtype == np.float32
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    # the same draws, with 1% of the elements multiplied by 20
    (a,) = datagen.streams(94, 1)
    (b,) = datagen.streams(94, 1)
    plain = datagen.activations(a, 64, 4096)
    out = datagen.activations(b, 64, 4096, outliers=True)
    scaled = out != plain
    frac = scaled.mean()
    assert 0.008 < frac < 0.012
    # the generator scales the float64 draw before its float32 cast: 20 times
    # the float32 value within one rounding of each
    ratio = out[scaled].astype(np.float64) / plain[scaled].astype(np.float64)
    assert np.all(np.abs(ratio - 20.0) <= 20.0 * 2.0 ** -23)


def test_workload_shapes():
    wq, wd, x = datagen.single_gemv()
    assert wq.shape == (896, 896) and wd.shape == (896, 28) and x.shape == (1, 896)
    layer = datagen.decode_layer_weights(0)
    for name, n, k in datagen.DECODE_LAYER:
        assert layer[name][0].shape == (n, k) and layer[name][1].shape == (n, k // 32)
    assert datagen.LM_HEAD == ("lm_head", 151936, 896)
    g = datagen.gate_up_inputs(n=64, k=256)
    assert g[0].shape == (64, 128) and g[1].shape == (64, 8) and g[4].shape == (8, 256)
    p = datagen.prefill_inputs(n=64, k=256, m=16)
    assert p[0].shape == (64, 128) and p[4].shape == (16, 256)
    assert (datagen.GATE_UP, datagen.PREFILL) == (dict(M=8, N=17408, K=5120), dict(M=1024, N=17408, K=5120))


def test_deterministic_and_distinct_copies():
    a = datagen.decode_layer_weights(3)
    b = datagen.decode_layer_weights(3)
    c = datagen.decode_layer_weights(4)
    for name, _, _ in datagen.DECODE_LAYER:
        assert np.array_equal(a[name][0], b[name][0]) and np.array_equal(a[name][1], b[name][1])
        assert not np.array_equal(a[name][0], c[name][0])
    x1, x2 = datagen.decode_activations(1), datagen.decode_activations(1)
    assert all(np.array_equal(x1[k], x2[k]) for k in (896, 4864))
    f1, f2 = datagen.q4_ffn_weights(0), datagen.q4_ffn_weights(1)
    assert not np.array_equal(f1["down"][0], f2["down"][0])

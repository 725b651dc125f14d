"""Host checks of two arithmetic facts the GPU quantiser relies on (IEEE
binary32 in numpy rounds as the GPU's VALU does, to nearest even).

The kernels form an int8 code as the low byte of fp32(t + 1.5 * 2**23),
t = fp32(x * s), and apply no clamp; these tests pin both steps against the
quantiser's definition (round half to even of the fp32 product, clamped to
[-128, 127]) without touching the GPU or the oracle.
"""
import numpy as np

MAGIC = np.float32(12582912.0)   # 1.5 * 2**23


def magic_code(t):
    """int8 code the kernels take: low byte of the sum's bits."""
    bits = (np.asarray(t, np.float32) + MAGIC).astype(np.float32).view(np.uint32)
    return (bits & 0xFF).astype(np.uint8).view(np.int8)


def test_magic_add_rounds_half_to_even_in_range():
    # every half-integer and its float neighbours in [-128, 127]
    base = np.arange(-256, 255, dtype=np.float64) / 2.0
    vals = [base.astype(np.float32)]
    for d in (1, 2):
        vals.append(np.nextafter(base.astype(np.float32), np.float32(np.inf)))
        vals.append(np.nextafter(base.astype(np.float32), np.float32(-np.inf)))
        base = np.nextafter(base, np.inf)
    rng = np.random.default_rng(7)
    vals.append(rng.uniform(-128.0, 127.4, 200_000).astype(np.float32))
    t = np.concatenate(vals)
    t = t[(t >= -128.0) & (t < 127.5)]
    want = np.clip(np.rint(t), -128, 127).astype(np.int8)
    np.testing.assert_array_equal(magic_code(t), want)


def test_scaled_tokens_never_need_the_clamp():
    """|fp32(x * fp32(127 / max(amax, 1e-5)))| < 127.5 whenever |x| <= amax:
    the extreme element lands on +-127 and nothing rounds past it."""
    rng = np.random.default_rng(11)
    amax = np.concatenate([
        np.float32(2.0) ** rng.uniform(-140, 127, 20_000).astype(np.float32),
        np.array([1e-5, 9.99e-6, 1e-30, 1.0, 127.0, 3.4e38], np.float32)]).astype(np.float32)
    denom = np.maximum(amax, np.float32(1e-5))
    s = (np.float32(127.0) / denom).astype(np.float32)
    for frac in (1.0, 0.999, 0.5, 0.123):
        for sign in (1.0, -1.0):
            x = (np.float32(sign * frac) * amax).astype(np.float32)
            t = (x * s).astype(np.float32)
            assert np.all(np.abs(t) < 127.5)
            want = np.clip(np.rint(t), -128, 127).astype(np.int8)
            np.testing.assert_array_equal(magic_code(t), want)
    # above the 1e-5 floor the element that sets the scale maps to 127 exactly
    big = amax >= np.float32(1e-5)
    t = (amax[big] * s[big]).astype(np.float32)
    assert t.size > 1000
    np.testing.assert_array_equal(magic_code(t), np.full(t.shape, 127, np.int8))

"""Host checks of the float32 identities the dot4 kernels rely on (no GPU).

The kernels start each integer dot chain from the bits of K = 1.5 * 2^23 and
scale the result with one fused multiply-add: fma(s, float(bits(K) + D), -K*s)
with s = d*sc.  That equals the rounded product s * float(D) exactly when
(1) bits(K) + D, read as a float32, is K + D for every reachable dot D, and
(2) -K*s is exact in float32 for every scale s the formats can hold.  Then the
fused operation computes s*(K + D) - K*s = s*D exactly and rounds it once,
which is what a multiply of s by the exactly converted D does.
"""
import numpy as np

K = np.float32(12582912.0)          # 1.5 * 2^23
K_BITS = 0x4B400000


def test_magic_offset_holds_every_dot():
    # q4_K chunk dots reach |D| <= 32 * 15 * 127; q6_K group dots 16 * 32 * 127;
    # the identity holds on all of |D| < 2^22.
    d = np.arange(-(1 << 22) + 1, 1 << 22, dtype=np.int64)
    as_float = (K_BITS + d).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(as_float, float(K) + d.astype(np.float64))
    assert 32 * 15 * 127 < (1 << 22) and 16 * 32 * 127 < (1 << 22)


def _all_finite_halves():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)].astype(np.float32)


def _exact_in_float32(x64):
    return np.array_equal(x64.astype(np.float32).astype(np.float64), x64)


def test_scaled_constant_is_exact_for_every_scale():
    d = _all_finite_halves()
    # q4_K: 6-bit sub-block scales; q6_K: signed 8-bit group scales
    for scales in (np.arange(0, 64), np.arange(-128, 128)):
        s = (d[:, None] * scales[None, :].astype(np.float32)).astype(np.float64)
        assert _exact_in_float32(s)                     # d*sc itself is exact
        assert _exact_in_float32(-float(K) * s)          # and so is -K*(d*sc)


def test_fused_form_equals_multiply_of_converted_dot():
    # The fused result rounds the exact s*D once; compare with float32 s*D
    # over random scales and dots (float64 holds s*D exactly: <= 17 + 17 bits).
    rng = np.random.default_rng(5)
    d = _all_finite_halves()
    s = (rng.choice(d, 200000) * rng.integers(-128, 128, 200000).astype(np.float32))
    dots = rng.integers(-65024, 65025, 200000)
    fused = (s.astype(np.float64) * (float(K) + dots) - float(K) * s.astype(np.float64))
    fused32 = fused.astype(np.float32)       # one rounding of the exact value
    plain = s * dots.astype(np.float32)      # float32 multiply, correctly rounded
    ok = np.isfinite(plain)
    assert np.array_equal(fused32[ok], plain[ok])

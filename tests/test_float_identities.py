"""CPU: the float32 identities the rotation's amax pass relies on to skip work
and stay bit-exact (no GPU needed; numpy float32 is IEEE round-to-nearest-even).

1. For finite a, b (no overflow): max(|fl(a + b)|, |fl(a - b)|) == fl(|a| + |b|).
   One of a + b, a - b has magnitude exactly |a| + |b| before rounding, the
   other one no larger, and rounding is monotone and sign-symmetric.
2. For c > 0: max_i fl(|y_i| * c) == fl(max_i |y_i| * c) (monotone rounding),
   so the 1/sqrt(128) normalisation can be applied to the maximum alone.
3. For finite values, the maximum of magnitudes as floats equals the maximum of
   the magnitude bit patterns (| 0x7fffffff) read back as a float.
"""
import numpy as np

F32 = np.float32
C = F32(float.fromhex("0x1.6a09e6p-4"))   # fl32(1/sqrt(128))


def _random_f32(n, rng):
    """Random float32 bit patterns over every finite exponent, plus ordinary
    values, half-integers (exact sums and ties), zeros of both signs and
    subnormals."""
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = np.where(np.isfinite(v), v, F32(1.0)).astype(F32)
    k = n // 16
    v[:k] = rng.standard_normal(k).astype(F32)
    v[k:2 * k] = (rng.integers(-64, 64, k) * 0.5).astype(F32)
    v[2 * k:2 * k + 64] = F32(0.0)
    v[2 * k + 64:2 * k + 128] = -F32(0.0)
    v[2 * k + 128:2 * k + 192] = (np.float32(1e-45) * rng.integers(1, 100, 64)).astype(F32)
    return v


def test_larger_of_sum_and_difference_is_sum_of_magnitudes():
    rng = np.random.default_rng(2024)
    n = 1 << 22
    a, b = _random_f32(n, rng), _random_f32(n, rng)
    # keep |a| + |b| finite (the transform never overflows in contract)
    a = np.where(np.abs(a) > F32(1e37), a * F32(1e-3), a).astype(F32)
    b = np.where(np.abs(b) > F32(1e37), b * F32(1e-3), b).astype(F32)
    with np.errstate(over="raise"):
        lhs = np.maximum(np.abs(a + b), np.abs(a - b))
        rhs = np.abs(a) + np.abs(b)
    assert lhs.dtype == np.float32 and rhs.dtype == np.float32
    assert np.array_equal(lhs.view(np.uint32), rhs.view(np.uint32))


def test_normalisation_commutes_with_the_maximum():
    rng = np.random.default_rng(2025)
    for _ in range(64):
        y = _random_f32(4096, rng)
        y = np.where(np.abs(y) > F32(1e37), y * F32(1e-3), y).astype(F32)
        per_value = np.max(np.abs(y) * C)
        once = F32(np.max(np.abs(y)) * C)
        assert per_value.view(np.uint32) == once.view(np.uint32)


def test_float_max_of_magnitudes_equals_bit_pattern_max():
    rng = np.random.default_rng(2026)
    y = _random_f32(1 << 20, rng).reshape(-1, 16)
    as_float = np.max(np.abs(y), axis=1)
    as_bits = np.max(y.view(np.uint32) & np.uint32(0x7FFFFFFF), axis=1).view(np.float32)
    assert np.array_equal(as_float.view(np.uint32), as_bits.view(np.uint32))

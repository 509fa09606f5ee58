"""The quantizers form fl32(a / b) as fl32(a * RN64(1 / b)) with one fp64 reciprocal
per bucket.  For fp32 a and b the fp64 product lies within 3 * 2^-53 (relative) of
a / b, while a quotient of two fp32 numbers that is not itself an fp32 number lies
more than 2^-49 (relative) from every halfway point between fp32 numbers, so the
two roundings agree.  This checks the identity against IEEE fp32 division (numpy)
on random operands over the whole exponent range (overflow, underflow, subnormal
operands and results), on divisors whose significand is close to 1 or to 2, and on
the quantizers' own quotient ranges."""
import numpy as np


def _pairs(rng, n, kind):
    ea = rng.integers(-149, 128, n)
    eb = rng.integers(-149, 128, n)
    ma = rng.integers(0, 1 << 23, n)
    mb = rng.integers(0, 1 << 23, n)
    if kind == 1:
        mb = (1 << 23) - 1 - rng.integers(0, 256, n)
    elif kind == 2:
        mb = rng.integers(0, 256, n)
    a = np.ldexp(1.0 + ma / 2.0 ** 23, ea).astype(np.float32)
    b = np.ldexp(1.0 + mb / 2.0 ** 23, eb).astype(np.float32)
    if kind == 3:                                    # (x - min) / step with t in [0, 255]
        b = rng.uniform(1e-6, 1e2, n).astype(np.float32)
        a = (rng.uniform(0, 255, n) * b).astype(np.float32)
    if kind == 4:                                    # |g| / norm with t in [0, 1]
        b = np.ldexp(rng.uniform(1, 2, n), rng.integers(-140, 60, n)).astype(np.float32)
        a = (b * rng.uniform(0, 1, n) ** 8).astype(np.float32)
    return a, b


def test_division_by_fp64_reciprocal_rounds_like_fp32_division():
    rng = np.random.default_rng(2024)
    for kind in range(5):
        a, b = _pairs(rng, 2_000_000, kind)
        with np.errstate(all="ignore"):
            ref = a / b
            got = (a.astype(np.float64) * (1.0 / b.astype(np.float64))).astype(np.float32)
        same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
        assert same.all(), f"kind {kind}: {a[~same][:3]} / {b[~same][:3]}"

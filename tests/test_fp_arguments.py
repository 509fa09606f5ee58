"""The floating-point arguments behind two fast paths of the kernels, checked on the
CPU with exact rational arithmetic (no GPU):

- the server's exact-sum tables: with every scale finite and the exponent fields of
  the nonzero scales spanning at most 29 - ceil(log2 W), the ordered fp64 sum of
  +-s_w and the sum regrouped by fours (and by batches of 16) are both the exact
  sum; one binade wider, an order can round;
- the QSGD / LoCo bucket norm from a plain fp64 sum of the squares: the plain sum
  (sequential per lane, then a butterfly over the 64 lanes) is within
  (n - 1) 2^-53 of the exact one, and wherever its square root lies more than
  2^-40 of itself from the midpoint between its two fp32 neighbours, it rounds to
  the same fp32 value as the square root of the correctly rounded sum.
"""
import math
from fractions import Fraction

import numpy as np


def _scales(rng, W, width, top=0):
    s = np.ldexp(rng.uniform(1, 2, W), rng.integers(top - width, top + 1, W)).astype(np.float32)
    s[0] = np.float32(np.ldexp(2.0 - 2.0 ** -23, top))               # full mantissa at the top
    if W > 1:
        s[-1] = np.float32(np.ldexp(1.0 + 2.0 ** -23, top - width))  # odd mantissa at the bottom
    return s.astype(np.float64)


def _ordered(v):
    acc = 0.0
    for x in v:
        acc = acc + x
    return acc


def _by_fours_in_batches(v):
    acc = 0.0
    for b0 in range(0, len(v), 16):
        for g0 in range(b0, min(b0 + 16, len(v)), 4):
            t = 0.0
            for x in v[g0:g0 + 4]:
                t = t + x
            acc = acc + t
    return acc


def test_exact_sum_bound_holds_at_its_widest_spread():
    for W in (2, 5, 16, 33, 100):
        lg = math.ceil(math.log2(W))
        rng = np.random.default_rng(W)
        for _ in range(12):
            s = _scales(rng, W, 29 - lg)
            for _ in range(60):
                v = rng.choice([-1.0, 1.0], W) * s
                exact = sum(Fraction(x) for x in v)
                assert Fraction(_ordered(v)) == exact
                assert Fraction(_by_fours_in_batches(v)) == exact


def test_one_binade_wider_an_order_can_round():
    # W = 16 allows a spread of 25: with 26, fifteen full mantissas at the top make a
    # partial sum near 30 (fp64 unit 2^-48), and the odd scale 26 binades below
    # (1 + 2^-23) 2^-26 needs the unit 2^-49: the ordered sum rounds
    top = float(np.float32(2.0 - 2.0 ** -23))
    low = float(np.float32((1.0 + 2.0 ** -23) * 2.0 ** -26))
    v = [top] * 15 + [low]
    assert Fraction(_ordered(v)) != sum(Fraction(x) for x in v)
    # and at the bound (spread 25) the same construction is exact
    low25 = float(np.float32((1.0 + 2.0 ** -23) * 2.0 ** -25))
    v = [top] * 15 + [low25]
    assert Fraction(_ordered(v)) == sum(Fraction(x) for x in v)


def _plain_norm(sq):
    """Per-lane sequential sums of 16 squares, then a butterfly over 64 lanes."""
    lanes = [_ordered(sq[16 * l:16 * l + 16]) for l in range(64)]
    o = 32
    while o:
        lanes = [lanes[l] + lanes[l ^ o] for l in range(64)]
        o >>= 1
    assert len(set(lanes)) == 1                                        # the same bits in every lane
    return lanes[0]


def _accept(r):
    f = np.float32(r)
    fb = int(f.view(np.uint32))
    nb = np.uint32(fb + 1 if float(f) <= r else fb - 1).view(np.float32)
    if not (math.isfinite(r) and np.isfinite(f) and np.isfinite(nb)):
        return None
    if r == 0.0:
        return np.float32(0.0)
    mid = 0.5 * (float(f) + float(nb))
    return f if abs(r - mid) > 2.0 ** -40 * r else None


def test_plain_sum_norm_is_within_its_bound_and_rounds_as_the_exact_one():
    rng = np.random.default_rng(11)
    accepted = 0
    for trial in range(120):
        kind = trial % 4
        if kind == 0:
            h = (rng.standard_normal(1024) * 1e-3).astype(np.float32)
        elif kind == 1:
            h = (rng.standard_normal(1024) * 10.0 ** rng.uniform(-20, 5, 1024)).astype(np.float32)
        elif kind == 2:
            h = rng.uniform(-1, 1, 1024).astype(np.float32)
            h[rng.random(1024) < 0.9] = 0.0
        else:
            h = (rng.standard_normal(1024) * 2.0 ** rng.integers(-60, 60)).astype(np.float32)
        sq = [float(x) * float(x) for x in h.astype(np.float64)]     # each square exact
        exact = sum(Fraction(x) for x in sq)
        plain = _plain_norm(sq)
        assert abs(Fraction(plain) - exact) <= Fraction(1023, 2 ** 53) * exact
        want = np.float32(math.sqrt(float(exact)))                  # fl32(sqrt(fl64(S)))
        got = _accept(math.sqrt(plain))
        if got is not None:
            accepted += 1
            assert got == want, (trial, got, want)
    assert accepted >= 110


def test_an_exact_tie_is_not_accepted():
    # (2^24 - 1)^2 + (2^13)^2 = (2^24 + 1)^2: the root is halfway between two fp32 values
    sq = [float(16777215) ** 2, float(8192) ** 2] + [0.0] * 1022
    assert _accept(math.sqrt(_plain_norm(sq))) is None

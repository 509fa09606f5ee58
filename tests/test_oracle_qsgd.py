"""Pins for the oracle's QSGD gradient quantizer and its W-worker decode/average.

Source: QSDP review (nubint.ai), "proposed method" (gradients take the standard
unbiased compressor of Alistarh et al. 2017); QSGD (Alistarh et al., NeurIPS 2017),
sec. 3.1: Q_s(v_i) = ||v||_2 sgn(v_i) xi_i / s with xi_i in {l, l + 1}, rounding up
with probability |v_i| s / ||v||_2 - l, so E[Q_s(v)] = v and the variance of one
coordinate is (||v|| / s)^2 p (1 - p).

Decoding reading: a code stands for the real number +-level * ||v|| / s, and the
average of W workers' values is the real number (sum_w +-level_w ||v_w||) / (s W);
the decoded fp32 value is that number rounded once (round to nearest even).

Pinned without retyping the oracle's steps: buckets whose ratios |v_i| s / ||v|| are
integers (Pythagorean-style vectors) must come out exactly and independently of the
seed; a lone non-zero goes to the top level and decodes to itself, for values over
the whole binary32 range; arbitrary codes and norms decode (W = 1) and average
(W = 2 ... 16) to the exact rational value rounded once to binary32, computed with
fractions.Fraction; the norm equals math.fsum in exact arithmetic; over 4096 seeds
the decoded mean is within 6 sigma of v and the mean squared error matches the
closed form; the round-up frequency of each element matches its p; averaging a
stream with its sign-flipped copy gives exactly 0.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def unpack4(codes, n):
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=1).reshape(-1)[:n]


def to_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rn32(q):
    """The binary32 number nearest the rational q (ties to even), as float32."""
    if q == 0:
        return np.float32(0.0)
    neg, a = q < 0, abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()      # 2^e <= a < 2^(e+2)
    if a >= Fraction(2) ** (e + 1):
        e += 1
    if a < Fraction(2) ** e:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)                        # subnormal spacing below 2^-126
    m, rem = divmod(a, ulp)
    m = int(m)
    if rem > ulp / 2 or (rem == ulp / 2 and m % 2 == 1):
        m += 1
    v = Fraction(m) * ulp
    if v >= Fraction(2) ** 128:
        return np.float32(-np.inf if neg else np.inf)
    return np.float32(-float(v) if neg else float(v))


def test_rn32_helper_against_numpy_on_exact_doubles():
    # on fp64 inputs numpy's float32 conversion is a single rounding: the helper must agree
    rng = np.random.default_rng(4)
    x = rng.standard_normal(4000) * 2.0 ** rng.integers(-160, 127, 4000)
    for v in x[np.abs(x) < 2.0 ** 127]:
        assert rn32(Fraction(float(v))) == np.float32(v)
    assert rn32(Fraction(3, 2 ** 150)) == np.float32(2.0 ** -148)   # tie between 1 and 2 subnormal steps: even
    assert rn32(Fraction(1, 2 ** 150)) == np.float32(0.0)             # half the smallest step: ties to 0


@pytest.mark.parametrize("as_bf16", [False, True])
def test_integer_ratio_buckets_are_exact(as_bf16):
    # 4-bit: s = 7; |(2, 3, 6)| = 7.   8-bit: s = 127; |(120, 41, 4, 4, 4)| = 127.
    g4 = np.array([2, -3, 6, 0, -2, 3, -6, 0], np.float32)
    g8 = np.array([120, -41, 4, -4, 4, 0, 0, 0, -120, 41, -4, 4, -4, 0, 0, 0], np.float32)
    for g, bits, bucket, levels in ((g4, 4, 4, [2, 3, 6, 0]), (g8, 8, 8, [120, 41, 4, 4, 4, 0, 0, 0])):
        s = 2 ** (bits - 1) - 1
        gin = to_bf16_bits(g) if as_bf16 else g
        for seed in (0, 1, 12345, 2 ** 63 + 7):
            codes, norms = oracle.qsgd_quantize(gin, bucket=bucket, bits=bits, seed=seed)
            np.testing.assert_array_equal(norms, np.full(g.size // bucket, s, np.float32))
            c = unpack4(codes, g.size) if bits == 4 else codes
            np.testing.assert_array_equal(c & s, np.tile(levels, g.size // bucket))
            np.testing.assert_array_equal(c >> (bits - 1), (g < 0).astype(np.uint8))
            y, yb = oracle.qsgd_reduce(codes, norms, g.size, bucket=bucket, bits=bits, want_bf16=True)
            np.testing.assert_array_equal(y, g)
            np.testing.assert_array_equal(yb, to_bf16_bits(g))


def test_lone_value_zero_bucket_signed_zero_and_padding():
    big, tiny = np.float32(-889 / 16), np.float32(889 * 2.0 ** -110)   # 889 = 7 * 127: level spacings exact
    g = np.array([0, 0, big, 0, 0, 0, 0, 0, -0.0, 0.0, -0.0, 0, tiny, 0, 0], np.float32)
    for bits in (4, 8):
        s = 2 ** (bits - 1) - 1
        codes, norms = oracle.qsgd_quantize(g, bucket=4, bits=bits, seed=3)
        np.testing.assert_array_equal(norms, np.array([-big, 0, 0, tiny], np.float32))
        c = unpack4(codes, g.size) if bits == 4 else codes
        expect = np.zeros(g.size, np.uint8)
        expect[2] = (1 << (bits - 1)) | s
        expect[12] = s
        np.testing.assert_array_equal(c, expect)
        if bits == 4:
            assert codes.size == 8 and codes[-1] >> 4 == 0          # pad nibble of the odd tail
        y, _ = oracle.qsgd_reduce(codes, norms, g.size, bucket=4, bits=bits)
        ref = np.zeros(g.size, np.float32)
        ref[2], ref[12] = big, tiny
        np.testing.assert_array_equal(y, ref)
        assert not np.signbit(y[8]) and not np.signbit(y[10])     # -0 is sent as +0


def random_norms(rng, W, nb, spread):
    """[W, nb] float32 norms: per bucket a base exponent over the binary32 range, each
    worker within `spread` binary orders of it (subnormal norms included)."""
    base = rng.integers(-150, 100, nb)
    e = base[None, :] + rng.integers(0, spread + 1, (W, nb))
    sig = rng.uniform(1.0, 2.0, (W, nb))
    return np.ldexp(sig, e).astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("W,spread", [(1, 0), (1, 200), (2, 18), (3, 18), (5, 18), (8, 18), (16, 18)])
def test_decode_is_exact_average_rounded_once(bits, W, spread):
    rng = np.random.default_rng(100 * W + bits + spread)
    s = 2 ** (bits - 1) - 1
    bucket, nb = 16, 24
    n = bucket * nb - 5                                   # ragged last bucket, odd n
    nbytes = (n + 1) // 2 if bits == 4 else n
    codes = rng.integers(0, 256, (W, nbytes), dtype=np.uint8)   # every byte is a valid code (pair)
    if bits == 4:
        codes[:, -1] &= 0x0F                               # pad nibble
    norms = random_norms(rng, W, nb, min(spread, 60))
    y, _ = oracle.qsgd_reduce(codes, norms, n, bucket=bucket, bits=bits)
    lv = np.stack([(unpack4(c, n) if bits == 4 else c[:n]) for c in codes]).astype(np.int64)
    for i in range(n):
        exact = sum(((-1) ** int(lv[w, i] >> (bits - 1))) * int(lv[w, i] & s) * Fraction(float(norms[w, i // bucket]))
                    for w in range(W)) / (s * W)
        assert y[i] == rn32(exact), (i, W, y[i], rn32(exact))


def test_lone_value_decodes_to_itself_over_the_whole_range():
    # one non-zero value v in a bucket: norm = |v|, level = s, decoded value s |v| / s = v
    rng = np.random.default_rng(21)
    k = 3000
    v = (rng.choice([-1.0, 1.0], k) * np.ldexp(rng.uniform(1.0, 2.0, k), rng.integers(-149, 127, k))).astype(np.float32)
    v = v[v != 0]
    bucket = 4
    g = np.zeros(bucket * v.size, np.float32)
    pos = rng.integers(0, bucket, v.size)
    g[np.arange(v.size) * bucket + pos] = v
    for bits in (4, 8):
        codes, norms = oracle.qsgd_quantize(g, bucket=bucket, bits=bits, seed=5)
        np.testing.assert_array_equal(norms, np.abs(v))
        y, _ = oracle.qsgd_reduce(codes, norms, g.size, bucket=bucket, bits=bits)
        np.testing.assert_array_equal(y, g)


def test_norm_is_the_rounded_exact_norm():
    rng = np.random.default_rng(8)
    n, bucket = 64 * 37, 64
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-20, 20, n)).astype(np.float32)
    _, norms = oracle.qsgd_quantize(g, bucket=bucket, bits=8, seed=0)
    for b in range(n // bucket):
        exact = math.fsum(float(v) ** 2 for v in g[b * bucket:(b + 1) * bucket].astype(np.float64))
        assert norms[b] == np.float32(math.sqrt(exact)), b


def test_slice_with_first_index_matches_whole_vector():
    rng = np.random.default_rng(9)
    g = (rng.standard_normal(5000) * 1e-3).astype(np.float32)
    for bits in (4, 8):
        full_c, full_n = oracle.qsgd_quantize(g, bucket=100, bits=bits, seed=77)
        part_c, part_n = oracle.qsgd_quantize(g[1200:3400], bucket=100, bits=bits, seed=77, first_index=1200)
        per = 2 if bits == 4 else 1
        np.testing.assert_array_equal(part_c, full_c[1200 // per:3400 // per])
        np.testing.assert_array_equal(part_n, full_n[12:34])


@pytest.mark.parametrize("bits", [4, 8])
def test_unbiased_and_variance_closed_form(bits):
    rng = np.random.default_rng(10 + bits)
    bucket, nb, S = 64, 6, 4096
    n = bucket * nb
    g = (rng.standard_normal(n) * 10.0 ** np.repeat(rng.uniform(-4, 0, nb), bucket)).astype(np.float32)
    s = 2 ** (bits - 1) - 1
    ys = np.zeros((S, n))
    ups = np.zeros(n)
    _, norms = oracle.qsgd_quantize(g, bucket=bucket, bits=bits, seed=0)
    nrm = np.repeat(norms.astype(np.float64), bucket)
    r = np.abs(g.astype(np.float64)) / nrm * s
    lvl, p = np.floor(r), r - np.floor(r)
    for seed in range(S):
        codes, _ = oracle.qsgd_quantize(g, bucket=bucket, bits=bits, seed=seed)
        ys[seed], _ = oracle.qsgd_reduce(codes, norms, n, bucket=bucket, bits=bits)
        c = unpack4(codes, n) if bits == 4 else codes
        ups += (c & s) > lvl
    var = (nrm / s) ** 2 * p * (1 - p)
    mean = ys.mean(axis=0)
    assert np.all(np.abs(mean - g) <= 6 * np.sqrt(var / S) + 1e-6 * nrm / s)
    mse = ((ys - g) ** 2).mean(axis=0)
    rel = ((mse - var) / np.maximum(var, 1e-300))[var > 0]
    assert abs(np.mean(rel)) < 0.05
    sd = np.sqrt(p * (1 - p) / S)
    assert np.all(np.abs(ups / S - p) <= 6 * sd + 1e-3)


def test_average_of_workers():
    rng = np.random.default_rng(11)
    g = (rng.standard_normal(3000) * 1e-2).astype(np.float32)
    for bits in (4, 8):
        c, nm = oracle.qsgd_quantize(g, bucket=1000, bits=bits, seed=5)
        flip = np.full_like(c, 0x88 if bits == 4 else 0x80)
        y1, _ = oracle.qsgd_reduce(c, nm, g.size, bucket=1000, bits=bits)
        y0, _ = oracle.qsgd_reduce(np.stack([c, c ^ flip]), np.stack([nm, nm]), g.size, bucket=1000, bits=bits)
        assert np.all(y0 == 0)
        y3, _ = oracle.qsgd_reduce(np.stack([c, c, c]), np.stack([nm, nm, nm]), g.size, bucket=1000, bits=bits)
        np.testing.assert_array_equal(y3, y1)
    # three integer-ratio workers: (2,3,6)/7 levels, averages known exactly
    a = np.array([2, 3, 6, 0], np.float32)
    ws = [a, -a, np.array([6, 2, 3, 0], np.float32)]
    cs, ns = zip(*(oracle.qsgd_quantize(w, bucket=4, bits=4, seed=0) for w in ws))
    y, _ = oracle.qsgd_reduce(np.stack(cs), np.stack(ns), 4, bucket=4, bits=4)
    np.testing.assert_array_equal(y, np.array([2, 2 / 3, 1, 0], np.float32))


def test_argument_errors():
    g = np.zeros(10, np.float32)
    for kw in (dict(bucket=3, bits=4), dict(bucket=4, bits=5), dict(bucket=0, bits=8)):
        with pytest.raises(Exception):
            oracle.qsgd_quantize(g, seed=0, **kw)

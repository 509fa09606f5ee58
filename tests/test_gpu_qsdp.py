"""GPU parity of the QSDP stochastic-rounding quantizer and dequantizer: codes,
bucket min/max and dequantized values bit-exact against the oracle, for 4- and
8-bit codes, fast (multiple of 4) and generic bucket sizes, ragged last buckets,
odd lengths (pad nibble), constant and signed-zero buckets."""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from gpu_helpers import DEV, host
from parity import assert_exact, say

pytestmark = pytest.mark.gpu


def bf16_dev(vals):
    return torch.as_tensor(np.asarray(vals, np.float32)).to(torch.bfloat16).to(DEV)


def quantize_both(xd, bucket, bits, seed):
    n = xd.numel()
    nb = (n + bucket - 1) // bucket
    nbytes = (n + 1) // 2 if bits == 4 else n
    codes = torch.zeros(max(nbytes, 1) + 16, dtype=torch.uint8, device=DEV)
    bmin = torch.zeros(max(nb, 1), dtype=torch.float32, device=DEV)
    bmax = torch.zeros(max(nb, 1), dtype=torch.float32, device=DEV)
    ob.qsdp_quantize(xd, bucket, bits, seed, codes, bmin, bmax)
    x = host(xd)
    rc, rmin, rmax = oracle.qsdp_quantize(x, bucket=bucket, bits=bits, seed=seed)
    torch.cuda.synchronize()
    gc = host(codes)
    assert_exact("codes", gc[:nbytes], rc)
    assert np.all(gc[nbytes:] == 0), "wrote past the end of the codes"
    assert_exact("bucket min", host(bmin)[:nb], rmin)
    assert_exact("bucket max", host(bmax)[:nb], rmax)
    y16 = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    y32 = torch.zeros(n, dtype=torch.float32, device=DEV)
    ob.qsdp_dequantize(codes, bmin, bmax, n, bucket, bits, y16, y32)
    r16, r32 = oracle.qsdp_dequantize(rc, rmin, rmax, n, bucket=bucket, bits=bits, want_f32=True)
    torch.cuda.synchronize()
    assert_exact("y f32", host(y32), r32)
    assert_exact("y bf16", host(y16), r16)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bucket", [1024, 1000, 1022, 64, 2])
def test_random_weights(bits, bucket):
    for n in (1, 7, 1024, 1025, 3 * 1024 + 256, 100_001):
        for seed in (0, 2 ** 40 + 5):
            say(f"qsdp bits={bits} bucket={bucket} n={n} seed={seed}")
            x = np.random.default_rng(n).standard_normal(n) * 0.02
            quantize_both(bf16_dev(x), bucket, bits, seed)


def test_generic_odd_bucket_8bit():
    x = np.random.default_rng(5).standard_normal(5003) * 0.02
    quantize_both(bf16_dev(x), 1023, 8, 11)


@pytest.mark.parametrize("bits", [4, 8])
def test_special_buckets(bits):
    vals = [0.5] * 1024 + [-0.0, 0.0] * 512 + [0.0, -0.0, 1.0, -1.0] * 256 + list(range(16)) * 64
    quantize_both(bf16_dev(vals), 1024, bits, 3)


def extreme_bf16(n, rng):
    """bf16 bit patterns over the whole finite exponent range (subnormals and signed
    zeros included; |x| < 2^126 so that every bucket's max - min stays finite), with
    buckets of tiny values only, a bucket whose minimum is +0 and one spanning
    2^-100 .. 2^100."""
    u = rng.integers(0, 1 << 16, n).astype(np.uint16)
    e = (u >> 7) & 0xFF
    big = e > 252
    u[big] = (u[big] & 0x807F) | (rng.integers(0, 253, int(big.sum())).astype(np.uint16) << 7)
    u[6 * 1024:7 * 1024] &= 0x80FF                                   # exponents 0..1: subnormal / tiny
    u[7 * 1024:8 * 1024] &= 0x7FFF                                   # non-negative ...
    u[7 * 1024 + 5] = 0                                              # ... with minimum +0
    ex = rng.integers(27, 228, 1024).astype(np.uint16)               # 2^-100 .. 2^100
    u[8 * 1024:9 * 1024] = (u[8 * 1024:9 * 1024] & 0x807F) | (ex << 7)
    return torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bucket", [1024, 1000, 64])
def test_extreme_exponents(bits, bucket):
    """The quotient (x - min) / step is formed from one fp64 reciprocal of the step per
    bucket; it must round exactly as the oracle's fp32 division on every range."""
    say(f"qsdp extreme exponents bits={bits} bucket={bucket}")
    quantize_both(extreme_bf16(16 * 1024 + 300, np.random.default_rng(bits * 1000 + bucket)), bucket, bits, 9)


def test_argument_errors():
    xd = bf16_dev(np.zeros(10))
    c = torch.zeros(16, dtype=torch.uint8, device=DEV)
    f = torch.zeros(4, dtype=torch.float32, device=DEV)
    for bad in (dict(bucket=1024, bits=5), dict(bucket=0, bits=8), dict(bucket=1023, bits=4)):
        with pytest.raises(ob.OnebitError):
            ob.qsdp_quantize(xd, bad["bucket"], bad["bits"], 0, c, f, f)

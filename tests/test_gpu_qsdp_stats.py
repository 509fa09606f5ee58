"""GPU 64-seed error statistic of the QSDP quantizer (the unbiasedness measurement).

Small size: the kernels' sums equal numpy fp64 sums over the oracle's dequantized
draws (same inputs, same seeds).  Full size (1.3e9 bf16 weights ~ N(0, 0.02),
buckets of 1024, 4-bit, seeds 0..63): the empirical mean squared error matches
the closed form mean_i Delta_i^2 p_i (1 - p_i) of stochastic rounding, and the
signed mean error is within statistical noise of 0.
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, host
from parity import say

pytestmark = pytest.mark.gpu


def _buffers(n, bucket, bits):
    nb = (n + bucket - 1) // bucket
    codes = torch.zeros((n + 1) // 2 if bits == 4 else n, dtype=torch.uint8, device=DEV)
    return codes, torch.zeros(nb, device=DEV), torch.zeros(nb, device=DEV)


def test_stats_match_numpy_on_oracle_draws():
    n, bucket, bits, S = 100_003, 1024, 4, 16
    x = torch.from_numpy((np.random.default_rng(3).standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16)
    xd = x.to(DEV)
    xh = x.view(torch.int16).numpy().view(np.uint16)
    xf = oracle.bf16_bits_to_f32(xh).astype(np.float64)
    codes, bmin, bmax = _buffers(n, bucket, bits)
    y = torch.zeros(n, device=DEV)
    ysum = torch.zeros(n, dtype=torch.float64, device=DEV)
    sums = torch.zeros(2, dtype=torch.float64, device=DEV)
    part = torch.zeros(2 * ob.QSDP_STATS_PARTIALS, dtype=torch.float64, device=DEV)
    ref1 = ref2 = 0.0
    ref_ysum = np.zeros(n)
    for s in range(S):
        ob.qsdp_quantize(xd, bucket, bits, s, codes, bmin, bmax)
        ob.qsdp_dequantize(codes, bmin, bmax, n, bucket, bits, None, y)
        ob.qsdp_error_stats(xd, y, ysum, sums, part)
        rc, rmn, rmx = oracle.qsdp_quantize(xh, bucket=bucket, bits=bits, seed=s)
        _, ry = oracle.qsdp_dequantize(rc, rmn, rmx, n, bucket=bucket, bits=bits, want_f32=True)
        d = ry.astype(np.float64) - xf
        ref1 += d.sum()
        ref2 += (d * d).sum()
        ref_ysum += ry
    mae = torch.zeros(1, dtype=torch.float64, device=DEV)
    ob.qsdp_mean_abs_error(xd, ysum, S, mae, part)
    torch.cuda.synchronize()
    got = host(sums)
    assert abs(got[0] - ref1) <= 1e-9 * np.abs(ref_ysum).sum() / S + 1e-12
    np.testing.assert_allclose(got[1], ref2, rtol=1e-12)
    np.testing.assert_allclose(host(ysum), ref_ysum, rtol=1e-15)
    np.testing.assert_allclose(host(mae)[0], np.abs(ref_ysum / S - xf).sum(), rtol=1e-12)


def test_stats_without_the_seed_sum():
    """ysum is optional: the sums alone, on an odd length (the last element is taken
    apart from the pairs)."""
    n, bucket, bits = 4099, 1024, 8
    x = torch.from_numpy((np.random.default_rng(8).standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16)
    xd = x.to(DEV)
    xh = x.view(torch.int16).numpy().view(np.uint16)
    codes, bmin, bmax = _buffers(n, bucket, bits)
    y = torch.zeros(n, device=DEV)
    sums = torch.zeros(2, dtype=torch.float64, device=DEV)
    part = torch.zeros(2 * ob.QSDP_STATS_PARTIALS, dtype=torch.float64, device=DEV)
    ob.qsdp_quantize(xd, bucket, bits, 5, codes, bmin, bmax)
    ob.qsdp_dequantize(codes, bmin, bmax, n, bucket, bits, None, y)
    ob.qsdp_error_stats(xd, y, None, sums, part)
    rc, rmn, rmx = oracle.qsdp_quantize(xh, bucket=bucket, bits=bits, seed=5)
    _, ry = oracle.qsdp_dequantize(rc, rmn, rmx, n, bucket=bucket, bits=bits, want_f32=True)
    d = ry.astype(np.float64) - oracle.bf16_bits_to_f32(xh).astype(np.float64)
    torch.cuda.synchronize()
    got = host(sums)
    assert abs(got[0] - d.sum()) <= 1e-12 * np.abs(ry).sum() + 1e-15
    np.testing.assert_allclose(got[1], (d * d).sum(), rtol=1e-12)


def test_64_seed_statistic_full_size():
    q = W.QsdpWorkload()
    bits, S = 4, q.seeds
    xq = W.qsdp_weights(q, device=DEV)
    codes, bmin, bmax = _buffers(q.n, q.bucket, bits)
    y = torch.zeros(q.n, device=DEV)
    ysum = torch.zeros(q.n, dtype=torch.float64, device=DEV)
    sums = torch.zeros(2, dtype=torch.float64, device=DEV)
    part = torch.zeros(2 * ob.QSDP_STATS_PARTIALS, dtype=torch.float64, device=DEV)
    for s in range(S):
        ob.qsdp_quantize(xq, q.bucket, bits, s, codes, bmin, bmax)
        ob.qsdp_dequantize(codes, bmin, bmax, q.n, q.bucket, bits, None, y)
        ob.qsdp_error_stats(xq, y, ysum, sums, part)
    mae = torch.zeros(1, dtype=torch.float64, device=DEV)
    ob.qsdp_mean_abs_error(xq, ysum, S, mae, part)
    torch.cuda.synchronize()
    s1, s2 = host(sums)
    # closed form of the per-element variance of stochastic rounding, fp64, chunked
    L = 2 ** bits - 1
    expected = 0.0
    step = 1 << 27
    for lo in range(0, q.n, step):
        hi = min(lo + step, q.n)
        xs = xq[lo:hi].double()
        b = torch.arange(lo, hi, device=DEV) // q.bucket
        mn = bmin[b].double()
        delta = ((bmax[b] - bmin[b]) / L).double()           # fl32 ops as the quantizer forms them
        t = torch.where(delta > 0, (xs - mn) / torch.where(delta > 0, delta, 1.0), torch.zeros_like(xs))
        p = t - torch.floor(t)
        expected += float((delta * delta * p * (1 - p)).sum())
        del xs, b, mn, delta, t, p
    mse = s2 / (S * q.n)
    mse_cf = expected / q.n
    bias = s1 / (S * q.n)
    sigma = np.sqrt(mse_cf / (S * q.n))
    say(f"  64-seed statistic: bias {bias:.3e} (sigma {sigma:.2e}), mse {mse:.6e} vs closed form {mse_cf:.6e}, "
        f"mean |avg_s y - x| {host(mae)[0] / q.n:.3e}")
    assert abs(mse / mse_cf - 1) < 1e-3
    assert abs(bias) < 6 * sigma

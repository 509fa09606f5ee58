"""Pins for the oracle's QSDP stochastic-rounding quantizer and its Philox stream.

Source: QSDP review ("Quantized Distributed Training of Large Models with
Convergence Guarantees"), "proposed method": each weight is rounded at random to
one of its two nearest quantization levels so that its expectation is the weight.
Philox4x32-10: Salmon et al., SC'11.

Pins:
  * values on the lattice are reproduced exactly for every seed (4- and 8-bit),
    which also fixes the nibble order of the 4-bit packing;
  * constant bucket -> code 0, min -> code 0; codes never exceed 2^b - 1;
  * unbiasedness by brute force over 2^16 seeds (mean within 5 sigma) and the
    variance closed form Delta^2 p (1 - p);
  * Philox against the authors' known-answer vectors and against two independent
    source implementations (rocRAND's and PyTorch's headers) for the
    (seed, element index) -> (key, counter, word) mapping.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def unpack_codes(codes, n, bits):
    if bits == 8:
        return codes[:n].astype(np.int64)
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=1).reshape(-1)[:n].astype(np.int64)


@pytest.mark.parametrize("bits", [4, 8])
def test_lattice_values_are_exact_for_every_seed(bits):
    L = 2 ** bits - 1
    bucket = L + 1
    vals = np.concatenate([np.arange(L + 1), np.arange(L + 1)[::-1], [3, 7, 0, L]]).astype(np.float32)
    x = bf16(vals)                                      # integers <= 255 are exact in bf16
    n = x.size
    for seed in (0, 1, 2 ** 40 + 3):
        codes, mn, mx = oracle.qsdp_quantize(x, bucket=bucket, bits=bits, seed=seed)
        got = unpack_codes(codes, n, bits)
        # every bucket spans [0, L] except the ragged last one ([0, L] too here)
        np.testing.assert_array_equal(got, vals.astype(np.int64))
        y16, y = oracle.qsdp_dequantize(codes, mn, mx, n, bucket=bucket, bits=bits, want_f32=True)
        np.testing.assert_array_equal(y, vals)
        np.testing.assert_array_equal(y16, x)
    if bits == 4:   # packing: even index in the low nibble, odd index in the high nibble
        np.testing.assert_array_equal(codes[:4], [(1 << 4) | 0, (3 << 4) | 2, (5 << 4) | 4, (7 << 4) | 6])


def test_degenerate_buckets_and_ragged_tail():
    # bucket 0 constant (Delta = 0), bucket 1 two-valued, last bucket ragged (odd n -> pad nibble)
    vals = [0.5] * 8 + [-1.0, 2.0] * 4 + [0.25, -0.75, 3.0]
    x = bf16(vals)
    n = x.size
    for bits in (4, 8):
        codes, mn, mx = oracle.qsdp_quantize(x, bucket=8, bits=bits, seed=5)
        c = unpack_codes(codes, n, bits)
        L = 2 ** bits - 1
        assert np.all(c[:8] == 0)
        np.testing.assert_array_equal(c[8:16], [0, L] * 4)        # min -> 0, max -> L (t == L exactly)
        assert c[16 + 1] == 0                                      # the minimum of the last bucket
        assert np.all(c <= L)
        np.testing.assert_array_equal(mn, np.float32([0.5, -1.0, -0.75]))
        np.testing.assert_array_equal(mx, np.float32([0.5, 2.0, 3.0]))
        y16, y = oracle.qsdp_dequantize(codes, mn, mx, n, bucket=8, bits=bits, want_f32=True)
        np.testing.assert_array_equal(y[:16], np.float32(vals[:16]))
    codes4, _, _ = oracle.qsdp_quantize(x, bucket=8, bits=4, seed=5)
    assert codes4.size == (n + 1) // 2 and (codes4[-1] >> 4) == 0  # pad nibble is zero


@pytest.mark.parametrize("bits", [4, 8])
def test_unbiased_and_variance_closed_form_brute_force(bits):
    rng = np.random.default_rng(bits)
    n = 12
    x = bf16(rng.standard_normal(n) * 0.02)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    S = 1 << 16
    ys = np.zeros((S, n))
    for s in range(S):
        codes, mn, mx = oracle.qsdp_quantize(x, bucket=n, bits=bits, seed=s)
        ys[s] = oracle.qsdp_dequantize(codes, mn, mx, n, bucket=n, bits=bits, want_f32=True)[1]
    L = 2 ** bits - 1
    delta = (float(mx[0]) - float(mn[0])) / L
    p = (xf - float(mn[0])) / delta
    p = p - np.floor(p)
    var = delta ** 2 * p * (1 - p)
    mean = ys.mean(axis=0)
    sigma = np.sqrt(var / S) + 1e-12
    assert np.all(np.abs(mean - xf) <= 5 * sigma + 1e-7 * delta), (mean - xf) / sigma
    emp_var = ((ys - xf) ** 2).mean(axis=0)
    ok = var > 1e-4 * delta ** 2
    np.testing.assert_allclose(emp_var[ok], var[ok], rtol=0.05)
    # values stay between neighbouring lattice points, up to the binary32 rounding of
    # y = min + code * Delta (relative to the magnitudes of both terms)
    lo = float(mn[0]) + np.floor((xf - float(mn[0])) / delta) * delta
    slack = 1e-6 * delta + 2.0 ** -21 * (abs(float(mn[0])) + np.abs(ys - float(mn[0])) + np.abs(ys))
    assert np.all(ys >= lo - slack) and np.all(ys <= lo + delta + slack)


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(w, 16) for w in line.split()])
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for r in rows:
        ctr, key, want = r[0:4], r[4:6], r[6:10]
        np.testing.assert_array_equal(oracle.philox4x32_10(key, ctr), np.array(want, np.uint32))


SAMPLES = [(0, 0), (0, 5), (0x0123456789ABCDEF, 7), (2 ** 64 - 1, 1_299_999_999), (42, 2 ** 34 + 3),
           (7, 4 * 0xFFFFFFFF + 2), (63, 1023), (1, 1_300_000_000 - 1)]


def _external(define, include):
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    src = os.path.join(HERE, "philox_ref.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "ref")
        cmd = [cxx, "-std=c++17", "-O1", f"-D{define}", *[f"-I{p}" for p in include], src, "-o", exe]
        if define == "USE_ROCRAND":
            cmd.insert(3, "-D__HIP_PLATFORM_AMD__")
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            pytest.skip(f"reference header did not compile: {r.stderr[-400:]}")
        inp = "\n".join(f"{s} {i}" for s, i in SAMPLES) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split()
    return [int(w, 16) for w in out]


@pytest.mark.parametrize("which", ["rocrand", "torch"])
def test_philox_element_stream_matches_independent_implementations(which):
    if which == "rocrand":
        inc = ["/opt/rocm/include"]
        if not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
            pytest.skip("rocRAND headers absent")
        got = _external("USE_ROCRAND", inc)
    else:
        inc = [os.path.join(os.path.dirname(torch.__file__), "include")]
        got = _external("USE_TORCH", inc)
    want = [oracle.qsdp_uniform(s, i) for s, i in SAMPLES]
    assert got == want


def test_signed_zero_order_and_slices():
    """Reading: min/max follow IEEE totalOrder (-0 < +0); a slice quantized with its
    global first index reproduces the same codes as the whole vector."""
    x = bf16([0.0, -0.0, 1.0, 2.0, -1.0, -0.0, 0.0, -2.0])
    codes, mn, mx = oracle.qsdp_quantize(x, bucket=4, bits=8, seed=3)
    assert np.signbit(mn[0]) and mn[0] == 0 and mx[0] == 2.0
    assert mn[1] == -2.0 and mx[1] == 0.0 and not np.signbit(mx[1])
    rng = np.random.default_rng(9)
    big = bf16(rng.standard_normal(4096) * 0.02)
    for bits in (4, 8):
        full, fmn, fmx = oracle.qsdp_quantize(big, bucket=1024, bits=bits, seed=77)
        part, pmn, pmx = oracle.qsdp_quantize(big[2048:3072], bucket=1024, bits=bits, seed=77, first_index=2048)
        per = 2 if bits == 4 else 1
        np.testing.assert_array_equal(part, full[2048 // per:3072 // per])
        assert pmn[0] == fmn[2] and pmx[0] == fmx[2]

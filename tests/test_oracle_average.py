"""Pins for the oracle's gradient average of the warmup phase (the full-precision
exchange: DeepSpeed 1-bit Adam guide, sec. 4, phase one, where Adam runs on the
gradient averaged over the workers).

Reading: the exact average of the W values, rounded once to binary32 (fp64 sum in
worker order, one division).  Pinned without retyping the oracle: one row is
returned unchanged; W copies of a row average to the row; a row and its negation
average to 0; bf16 rows (8 significant bits, so their fp64 sums are exact) and fp32
rows whose exponents lie within 20 of each other average to the exact rational mean
rounded once (fractions.Fraction), for W = 2, 3, 5, 8, 16.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from test_oracle_qsgd import rn32


def test_one_row_copies_and_negation():
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(1000) * 10.0 ** rng.uniform(-30, 30, 1000)).astype(np.float32)
    np.testing.assert_array_equal(oracle.average_rows(g[None, :]), g)
    for W in (2, 3, 7, 16):
        np.testing.assert_array_equal(oracle.average_rows(np.stack([g] * W)), g)
    z = oracle.average_rows(np.stack([g, -g]))
    assert np.all(z == 0)


@pytest.mark.parametrize("W", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("bf16", [False, True])
def test_exact_mean_rounded_once(W, bf16):
    rng = np.random.default_rng(10 * W + bf16)
    n = 400
    base = rng.integers(-120, 100, n)
    e = base[None, :] + rng.integers(0, 21, (W, n))
    g = (rng.choice([-1.0, 1.0], (W, n)) * np.ldexp(rng.uniform(1, 2, (W, n)), e)).astype(np.float32)
    if bf16:
        g = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
        out = oracle.average_rows(torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    else:
        out = oracle.average_rows(g)
    for i in range(n):
        exact = sum(Fraction(float(g[w, i])) for w in range(W)) / W
        assert out[i] == rn32(exact), (i, out[i], rn32(exact))

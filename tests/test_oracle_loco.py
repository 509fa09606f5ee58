"""Pins for the oracle's LoCo-style compensated gradient quantizer.

Source: shd-paper.top summary of LoCo (core points; method details, steps 2-4): the
gradient is compensated, before compression, by a moving average of the historical
compensation errors.  The page gives no formula, window or weights, so the step is
a reading of that description (parity unpinned as to the method itself); what is pinned is
the reading's own structure:

- beta = 0 and a zero average: the codes are the plain QSGD codes of g and the new
  average is the compression error g - decode(codes) (the pinned QSGD decode);
- beta = 0 over several steps is error feedback: sum_t y_t + e_T - e_0 = sum_t g_t
  up to the rounding of the two fp32 additions per step;
- for beta in (0, 1) the average equals its closed form
  beta^T e_0 + sum_t (1 - beta) beta^(T-t) (h_t - y_t), within the rounding of the
  recursion, where h_t = g_t + e_(t-1) and y_t is the decode of step t's codes.
"""
import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24


def grads(n, steps, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -2)).astype(np.float32) for _ in range(steps)]


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_average_is_plain_qsgd_and_error(bits):
    g = grads(5000, 1, 1)[0]
    e = np.zeros_like(g)
    c, nm = oracle.loco_quantize(g, e, bucket=1000, bits=bits, beta=0.0, seed=11)
    rc, rn = oracle.qsgd_quantize(g, bucket=1000, bits=bits, seed=11)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(nm, rn)
    y, _ = oracle.qsgd_reduce(rc, rn, g.size, bucket=1000, bits=bits)
    np.testing.assert_array_equal(e, g - y)
    gb = torch.from_numpy(g).to(torch.bfloat16)
    e2 = np.zeros_like(g)
    c2, _ = oracle.loco_quantize(gb.view(torch.int16).numpy().view(np.uint16), e2, bucket=1000, bits=bits, beta=0.0,
                                 seed=11)
    rc2, _ = oracle.qsgd_quantize(gb.float().numpy(), bucket=1000, bits=bits, seed=11)
    np.testing.assert_array_equal(c2, rc2)


def run(gs, e0, beta, bits, bucket=512):
    e = e0.copy()
    hs, ys, es = [], [], [e0.astype(np.float64)]
    for t, g in enumerate(gs):
        h = g + e                                           # the compensated gradient, one fp32 add
        c, nm = oracle.loco_quantize(g, e, bucket=bucket, bits=bits, beta=beta, seed=100 + t)
        y, _ = oracle.qsgd_reduce(c, nm, g.size, bucket=bucket, bits=bits)
        hs.append(h.astype(np.float64))
        ys.append(y.astype(np.float64))
        es.append(e.astype(np.float64))
    return hs, ys, es


@pytest.mark.parametrize("bits", [4, 8])
def test_beta_zero_is_error_feedback(bits):
    n, T = 4096, 6
    gs = grads(n, T, 2)
    e0 = (np.random.default_rng(3).standard_normal(n) * 1e-4).astype(np.float32)
    hs, ys, es = run(gs, e0, 0.0, bits)
    lhs = sum(ys) + es[-1] - es[0]
    rhs = sum(g.astype(np.float64) for g in gs)
    bound = U * sum(np.abs(h) + np.abs(e) for h, e in zip(hs, es[1:]))
    assert np.all(np.abs(lhs - rhs) <= bound * 1.0001 + 1e-300)


@pytest.mark.parametrize("beta", [0.5, 0.9])
def test_moving_average_closed_form(beta):
    n, T, bits = 4096, 6, 4
    gs = grads(n, T, 4)
    e0 = (np.random.default_rng(5).standard_normal(n) * 1e-4).astype(np.float32)
    hs, ys, es = run(gs, e0, beta, bits)
    b32, ob32 = float(np.float32(beta)), float(np.float32(1.0 - beta))
    closed = b32 ** T * es[0]
    bound = np.zeros(n)
    for t in range(T):
        closed = closed + ob32 * b32 ** (T - 1 - t) * (hs[t] - ys[t])
        # each recursion step rounds three times: beta*e, (1-beta)*(h-y) with h-y, and the sum
        bound += b32 ** (T - 1 - t) * 3 * U * (b32 * np.abs(es[t]) + ob32 * np.abs(hs[t] - ys[t]) + np.abs(es[t + 1]))
    assert np.all(np.abs(es[-1] - closed) <= bound * 1.0001 + 1e-300)


def test_exact_levels_leave_zero_average_unchanged():
    g = np.tile(np.array([2, -3, 6, 0], np.float32), 256)       # every bucket (2, -3, 6, 0): exact 4-bit levels
    for beta in (0.0, 0.5):
        e = np.zeros_like(g)
        for t in range(3):
            oracle.loco_quantize(g, e, bucket=4, bits=4, beta=beta, seed=t)
            assert np.all(e == 0)

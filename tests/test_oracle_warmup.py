"""Pins for the oracle's warmup (full-precision Adam) step.

Pinned against: the closed form of Adam under a constant gradient, and torch's own
Adam / AdamW on the CPU (bias-corrected; AdamW for decoupled weight decay).
Source of the step: DeepSpeed 1-bit Adam guide, sec. 4 (phase one is standard
Adam) and sec. 3.4 (lr, betas, eps, weight_decay, bias_correction).
"""
import numpy as np
import pytest
import torch

import oracle

H = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _x_tol(x_ref, x_prev):
    return 1e-5 * np.maximum(np.abs(x_ref), np.abs(x_ref - x_prev)) + 1e-30


@pytest.mark.parametrize("bias_correction", [False, True])
def test_constant_gradient_closed_form(bias_correction):
    rng = np.random.default_rng(11)
    n, T = 4099, 12
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[:3] = [0.0, 1e-30, -2.5]
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    x, m, v = x0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    # Each hyperparameter reaches the arithmetic as one binary32 value; 1-beta is
    # rounded from binary64, so beta and 1-beta are two separate constants here.
    b1, b2, eps, lr = (float(np.float32(H[k])) for k in ("beta1", "beta2", "eps", "lr"))
    ob1, ob2 = float(np.float32(1 - H["beta1"])), float(np.float32(1 - H["beta2"]))
    gd = g.astype(np.float64)
    x_cf = x0.astype(np.float64)
    for t in range(1, T + 1):
        oracle.adam_warmup_step(x, m, v, g, weight_decay=0.0, bias_correction=bias_correction, step=t, **H)
        # m_t = b1 m_{t-1} + ob1 g from 0 (geometric series); likewise v_t with g^2
        m_cf = ob1 * (1 - b1 ** t) / (1 - b1) * gd
        v_cf = ob2 * (1 - b2 ** t) / (1 - b2) * gd * gd
        np.testing.assert_allclose(m, m_cf, rtol=2e-6, atol=0)
        np.testing.assert_allclose(v, v_cf, rtol=4e-6, atol=1e-44)  # g^2 of 1e-30 underflows in fp32
        if bias_correction:
            bc1, bc2 = float(np.float32(1 - H["beta1"] ** t)), float(np.float32(1 - H["beta2"] ** t))
            step = lr * (m_cf / bc1) / (np.sqrt(v_cf / bc2) + eps)   # ~ lr g / (|g| + eps)
        else:
            step = lr * m_cf / (np.sqrt(v_cf) + eps)
        x_prev = x_cf
        x_cf = x_cf - step
        assert np.all(np.abs(x - x_cf) <= _x_tol(x_cf, x_prev) + 1e-9 * t)


def _torch_run(opt_cls, wd, steps, seed=5, n=3001):
    rng = np.random.default_rng(seed)
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(n) * 10 ** rng.uniform(-4, -1)).astype(np.float32) for _ in range(steps)]
    p = torch.nn.Parameter(torch.from_numpy(x0.copy()))
    opt = opt_cls([p], lr=H["lr"], betas=(H["beta1"], H["beta2"]), eps=H["eps"], weight_decay=wd, foreach=False)
    ref = []
    for gi in grads:
        p.grad = torch.from_numpy(gi.copy())
        x_prev = p.detach().numpy().copy()
        opt.step()
        st = opt.state[p]
        ref.append((p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy(),
                    x_prev))
    return x0, grads, ref


@pytest.mark.parametrize("opt_cls,wd", [(torch.optim.Adam, 0.0), (torch.optim.AdamW, 0.01)])
def test_matches_torch(opt_cls, wd):
    """Same trajectory as torch's Adam/AdamW, up to propagated binary32 rounding.

    torch forms m by lerp (m + (1-b1)(g - m)), so the two sides round differently;
    where b1*m and (1-b1)*g cancel the difference is relative to those terms and it
    decays by b1 per step afterwards.  The bounds below track exactly that.
    """
    u = 2.0 ** -23
    b1, lr, eps = H["beta1"], H["lr"], H["eps"]
    x0, grads, ref = _torch_run(opt_cls, wd, steps=8)
    x, m, v = x0.copy(), np.zeros_like(x0), np.zeros_like(x0)
    tol_m = np.zeros(x0.size)
    tol_x = np.zeros(x0.size)
    for t, (gi, (xr, mr, vr, xp)) in enumerate(zip(grads, ref), start=1):
        m_prev = m.astype(np.float64)
        oracle.adam_warmup_step(x, m, v, gi, weight_decay=wd, bias_correction=True, step=t, **H)
        tol_m = b1 * tol_m + 4 * u * (np.abs(b1 * m_prev) + np.abs((1 - b1) * gi) + np.abs(m))
        assert np.all(np.abs(m.astype(np.float64) - mr) <= tol_m)
        np.testing.assert_allclose(v, vr, rtol=1e-5, atol=1e-30)
        bc1, bc2 = 1 - b1 ** t, 1 - H["beta2"] ** t
        denom = np.sqrt(v.astype(np.float64) / bc2) + eps
        step = lr * np.abs(m) / bc1 / denom
        tol_x = tol_x * (1 + lr * wd) + lr * tol_m / bc1 / denom + 1e-5 * step + 4 * u * np.abs(x)
        assert np.all(np.abs(x.astype(np.float64) - xr) <= tol_x), np.max(np.abs(x - xr) - tol_x)


def test_bf16_gradient_is_exact_widening():
    rng = np.random.default_rng(3)
    g32 = torch.from_numpy((rng.standard_normal(777) * 1e-2).astype(np.float32)).to(torch.bfloat16)
    g_bits = g32.view(torch.int16).numpy().view(np.uint16)
    g_wide = g32.float().numpy()                              # torch's widening
    np.testing.assert_array_equal(oracle.bf16_bits_to_f32(g_bits), g_wide)
    a = [np.zeros(777, np.float32) for _ in range(3)]
    b = [np.zeros(777, np.float32) for _ in range(3)]
    oracle.adam_warmup_step(*a, g_bits, weight_decay=0.0, bias_correction=False, step=1, **H)
    oracle.adam_warmup_step(*b, g_wide, weight_decay=0.0, bias_correction=False, step=1, **H)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)


def test_f16_gradient_is_exact_widening():
    """fp16 gradients enter as their exact binary32 values, subnormals included:
    2^-24 (the smallest fp16 subnormal), 65504 (the largest finite), -0."""
    special = np.array([2.0 ** -24, 3 * 2.0 ** -24, 65504.0, -0.0, 2.0 ** -14, -1.5], np.float64)
    g16 = np.concatenate([special.astype(np.float16),
                          (np.random.default_rng(4).standard_normal(771) * 1e-4).astype(np.float16)])
    g_wide = torch.from_numpy(g16).float().numpy()
    np.testing.assert_array_equal(g_wide[:6], special.astype(np.float32))
    n = g16.size
    a = [np.zeros(n, np.float32) for _ in range(3)]
    b = [np.zeros(n, np.float32) for _ in range(3)]
    oracle.adam_warmup_step(*a, g16, weight_decay=0.0, bias_correction=False, step=1, **H)
    oracle.adam_warmup_step(*b, g_wide, weight_decay=0.0, bias_correction=False, step=1, **H)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)
    off = np.array([0, 300, n], np.int64)
    r16 = oracle.compress_update(off, g16, np.zeros(n, np.float32), np.zeros(n, np.float32), beta1=0.0)
    r32 = oracle.compress_update(off, g_wide, np.zeros(n, np.float32), np.zeros(n, np.float32), beta1=0.0)
    for u, w in zip(r16[:2], r32[:2]):
        np.testing.assert_array_equal(u, w)
    assert np.signbit(oracle.decompress(off, r16[0], r16[1])[3]) == 0   # sign(-0) = +1

"""GPU parity of the 1-bit Adam driver (error_compensated_bit_amd.optimizer) against the
oracle run through the same phases: full-precision warmup up to freeze_step, then
compressed steps with v frozen; a checkpoint reload in the compressed phase (m, v and
the step kept, the error restarted from zero); masked tensors pinned at zero."""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import workloads as W
from error_compensated_bit_amd.optimizer import OneBitAdam
from gpu_helpers import DEV, host
from parity import assert_bits_exact, assert_exact, check_scales, check_x, say

pytestmark = pytest.mark.gpu


class OracleAdam:
    """The oracle driven through the same phases on host arrays."""

    def __init__(self, x, chunk_off, tensor_off, tensor_keep, hp, freeze_step):
        self.x, self.m, self.v, self.e = x.copy(), np.zeros_like(x), np.zeros_like(x), np.zeros_like(x)
        self.off, self.to, self.tk, self.hp, self.freeze = chunk_off, tensor_off, tensor_keep, hp, freeze_step
        self.t = 0
        self.bits = self.scales = None

    def step(self, g):
        self.t += 1
        hp = self.hp
        if self.t <= self.freeze:
            oracle.adam_warmup_step(self.x, self.m, self.v, g, lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"],
                                    eps=hp["eps"], weight_decay=hp["weight_decay"],
                                    bias_correction=hp["bias_correction"], step=self.t)
        else:
            self.bits, self.scales, _ = oracle.compress_update(
                self.off, g, self.m, self.e, self.v, self.x, tensor_off=self.to, tensor_keep=self.tk, lr=hp["lr"],
                beta1=hp["beta1"], eps=hp["eps"], weight_decay=hp["weight_decay"])


def check(tag, o, r, x_prev):
    torch.cuda.synchronize()
    say(f"  {tag}")
    assert_exact(f"{tag} m", host(o.m), r.m)
    assert_exact(f"{tag} v", host(o.v), r.v)
    check_x(f"{tag} x", host(o.x), r.x, x_prev)
    if r.bits is not None and o.frozen:
        assert_bits_exact(f"{tag} bits", host(o.bits)[:r.bits.size].view(np.uint32), r.bits)
        assert check_scales(f"{tag} scales", host(o.scales)[:r.scales.size], r.scales) == 0
        assert_exact(f"{tag} e", host(o.e), r.e)


@pytest.mark.parametrize("bias_correction", [False, True])
def test_tiny_workload_through_the_driver(bias_correction):
    """1,048,576 params, one chunk: 5 warmup steps, then compressed steps; at step 7 a
    checkpoint is saved and loaded into a fresh driver, which continues to step 10."""
    wl = W.tiny()
    hp = dict(W.HYPER, bias_correction=bias_correction)
    x0 = W.init_state(wl)[0].numpy().copy()
    o = OneBitAdam(torch.from_numpy(x0.copy()).to(DEV), lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                   eps=hp["eps"], weight_decay=hp["weight_decay"], bias_correction=bias_correction, freeze_step=5)
    r = OracleAdam(x0, wl.chunk_off, None, None, hp, 5)
    for t in range(1, 11):
        g = W.gradient(wl, t).numpy()
        x_prev = r.x.copy()
        o.step(torch.from_numpy(g).to(DEV))
        r.step(g)
        check(f"bias_correction={bias_correction} step {t}", o, r, x_prev)
        if t == 7:
            sd = o.state_dict()
            o = OneBitAdam(o.x, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                           weight_decay=hp["weight_decay"], bias_correction=bias_correction, freeze_step=5)
            o.e.fill_(1.0)
            o.load_state_dict(sd)
            r.e[:] = 0.0
            assert o.frozen and torch.count_nonzero(o.e) == 0


def test_masked_tensors_through_the_driver():
    sizes = [1000, 2000, 1099, 4096 + 3]
    to = W.offsets_from_sizes(sizes)
    keep = np.array([1, 0, 1, 0], np.uint8)
    n = int(to[-1])
    rng = np.random.default_rng(11)
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(W.HYPER)
    o = OneBitAdam(torch.from_numpy(x0.copy()).to(DEV), tensor_offsets=to, tensor_keep=keep, lr=hp["lr"],
                   betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=0.0,
                   bias_correction=hp["bias_correction"], freeze_step=2)
    r = OracleAdam(x0, to, to, keep, dict(hp, weight_decay=0.0), 2)
    masked = np.repeat(keep == 0, np.diff(to))
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        g[masked] = 0.0
        x_prev = r.x.copy()
        o.step(torch.from_numpy(g).to(DEV))
        r.step(g)
        check(f"masked tensors step {t}", o, r, x_prev)
        if t > 2:
            assert np.all(host(o.m)[masked] == 0) and np.all(host(o.e)[masked] == 0)
            assert np.array_equal(host(o.x)[masked], x_prev[masked])


def test_driver_raises_on_a_failed_wait_and_recovers_from_a_checkpoint():
    """The host sets the workspace's error word before a compressed step (as a wait
    that gave up in an earlier step would have left it): every bounded wait of that
    step gives up at once and its kernels still exit; the driver reads the word after
    the step, re-initializes the workspace and raises WaitTimeout.  Reloading the
    checkpoint taken before that step and repeating it matches the oracle."""
    from error_compensated_bit_amd.optimizer import WaitTimeout
    off = W.fixed_chunks(3 << 20, 1 << 20)
    n = int(off[-1])
    rng = np.random.default_rng(12)
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(W.HYPER)
    kw = dict(chunk_offsets=off, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=0.0,
              freeze_step=1)
    o = OneBitAdam(torch.from_numpy(x0.copy()).to(DEV), **kw)
    r = OracleAdam(x0, off, None, None, dict(hp, weight_decay=0.0), 1)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(3)]
    for t in range(2):
        x_prev = r.x.copy()
        o.step(torch.from_numpy(grads[t]).to(DEV))
        r.step(grads[t])
        check(f"step {t + 1}", o, r, x_prev)
    sd = o.state_dict()
    x_saved = o.x.clone()
    o.workspace[0] = 2
    with pytest.raises(WaitTimeout):
        o.step(torch.from_numpy(grads[2]).to(DEV))
    say("  forced error word: WaitTimeout raised")
    assert int(o.workspace[0].item()) == 0
    o.x.copy_(x_saved)
    o.load_state_dict(sd)
    r.e[:] = 0.0
    x_prev = r.x.copy()
    o.step(torch.from_numpy(grads[2]).to(DEV))
    r.step(grads[2])
    check("step 3 after the reload", o, r, x_prev)


def test_zero_one_adam_variance_schedule_through_the_driver():
    """0/1 Adam's adaptive variance freezing as read here (the guide names only the
    method and its parameters; parity unpinned as to the method): var_freeze_step = 10,
    var_update_scaler = 2, so v is updated at steps 1, 2, 3, 5, 7 (spacings 1, 1, 2, 2,
    4) by full-precision Adam steps and every other step is the compressed step with
    the current v.  The driver matches the oracle run through that schedule for 14
    steps: m, v and the error bit for bit, x within tolerance."""
    from error_compensated_bit_amd.optimizer import ZeroOneAdam
    off = W.offsets_from_sizes([5000, 2 * 4096 + 1, 70001])
    n = int(off[-1])
    rng = np.random.default_rng(13)
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = dict(W.HYPER, weight_decay=0.01)
    o = ZeroOneAdam(torch.from_numpy(x0.copy()).to(DEV), chunk_offsets=off, lr=hp["lr"],
                    betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"],
                    var_freeze_step=10, var_update_scaler=2)
    var_steps = {1, 2, 3, 5, 7}
    x, m, v, e = x0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 15):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        x_prev = x.copy()
        o.step(torch.from_numpy(g).to(DEV))
        if t in var_steps:
            oracle.adam_warmup_step(x, m, v, g, lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                    weight_decay=hp["weight_decay"], bias_correction=False, step=t)
        else:
            oracle.compress_update(off, g, m, e, v, x, lr=hp["lr"], beta1=hp["beta1"], eps=hp["eps"],
                                   weight_decay=hp["weight_decay"])
        torch.cuda.synchronize()
        tag = f"0/1 Adam step {t} ({'variance update' if t in var_steps else 'compressed'})"
        say(f"  {tag}")
        assert_exact(f"{tag} m", host(o.m), m)
        assert_exact(f"{tag} v", host(o.v), v)
        assert_exact(f"{tag} e", host(o.e), e)
        check_x(f"{tag} x", host(o.x), x, x_prev)

"""Host logic of the 1-bit Adam driver (no GPU): which library call each step makes,
the freeze boundary, the step numbers handed to the warmup, and the error reset on
checkpoint load.  The library calls are replaced by recorders; the tensors are CPU
tensors that no kernel touches."""
import numpy as np
import pytest
import torch

from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import optimizer as opt


@pytest.fixture
def calls(monkeypatch):
    log = []
    monkeypatch.setattr(ob, "onebit_plan_create", lambda co, to=None, tk=None: ("plan", np.asarray(co).tolist()))
    monkeypatch.setattr(ob, "onebit_plan_words", lambda p: 3)
    monkeypatch.setattr(ob, "onebit_plan_chunks", lambda p: 2)
    monkeypatch.setattr(ob, "onebit_plan_workspace_bytes", lambda p: 64)

    def warm(x, m, v, g, **k):
        log.append(("warmup", k["step"], k["bias_correction"], k["beta2"]))

    def comp(plan, g, m, e, v, x, xb, bits, scales, **k):
        assert e is not None and v is not None and x is not None and xb is None
        log.append(("compress", plan[1], k["beta1"], k["lr"]))

    def status(ws, stream=None):
        log.append(("status",))
        return int(ws[0])

    def init(ws, stream=None):
        log.append(("init",))
        ws.zero_()

    monkeypatch.setattr(ob, "onebit_adam_warmup_step", warm)
    monkeypatch.setattr(ob, "onebit_compress_update", comp)
    monkeypatch.setattr(ob, "onebit_workspace_status", status)
    monkeypatch.setattr(ob, "onebit_workspace_init", init)
    return log


def test_warmup_then_compressed_steps(calls):
    x = torch.zeros(10)
    o = opt.OneBitAdam(x, chunk_offsets=[0, 4, 10], lr=2e-3, betas=(0.8, 0.99), freeze_step=3,
                       bias_correction=False)
    assert not o.frozen
    for _ in range(5):
        o.step(torch.zeros(10))
    assert o.frozen and o.step_count == 5
    assert calls == [("warmup", 1, False, 0.99), ("warmup", 2, False, 0.99), ("warmup", 3, False, 0.99),
                     ("compress", [0, 4, 10], 0.8, 2e-3), ("status",), ("compress", [0, 4, 10], 0.8, 2e-3),
                     ("status",)]
    assert o.bits.numel() == 3 and o.scales.numel() == 2 and o.workspace.numel() == 8


def test_default_chunks_follow_tensors_then_whole_vector(calls):
    o = opt.OneBitAdam(torch.zeros(6), tensor_offsets=[0, 2, 6], tensor_keep=[1, 0], freeze_step=0)
    o.step(torch.zeros(6))
    assert calls == [("compress", [0, 2, 6], 0.9, 1e-3), ("status",)]
    calls.clear()
    o = opt.OneBitAdam(torch.zeros(6), freeze_step=0)
    o.step(torch.zeros(6))
    assert calls == [("compress", [0, 6], 0.9, 1e-3), ("status",)]


def test_checkpoint_keeps_moments_and_resets_error(calls):
    o = opt.OneBitAdam(torch.zeros(4), freeze_step=2)
    for _ in range(3):
        o.step(torch.zeros(4))
    o.m.fill_(1.0)
    o.v.fill_(2.0)
    o.e.fill_(3.0)
    sd = o.state_dict()
    assert set(sd) == {"step", "exp_avg", "exp_avg_sq"} and sd["step"] == 3
    p = opt.OneBitAdam(torch.zeros(4), freeze_step=2)
    p.e.fill_(5.0)
    p.load_state_dict(sd)
    assert p.step_count == 3 and p.frozen
    assert torch.equal(p.m, torch.ones(4)) and torch.equal(p.v, torch.full((4,), 2.0))
    assert torch.equal(p.e, torch.zeros(4))
    calls.clear()
    p.step(torch.zeros(4))
    assert calls[0][0] == "compress"


def test_rejects_bad_arguments(calls):
    with pytest.raises(TypeError):
        opt.OneBitAdam(torch.zeros(4, dtype=torch.float64))
    with pytest.raises(TypeError):
        opt.OneBitAdam(torch.zeros(2, 2))
    with pytest.raises(ValueError):
        opt.OneBitAdam(torch.zeros(4), chunk_offsets=[0, 3])
    with pytest.raises(ValueError):
        opt.OneBitAdam(torch.zeros(4), freeze_step=-1)
    o = opt.OneBitAdam(torch.zeros(4))
    with pytest.raises(ValueError):
        o.step(torch.zeros(5))
    assert calls == []


def test_bias_correction_is_off_by_default(calls):
    o = opt.OneBitAdam(torch.zeros(4), freeze_step=1)
    o.step(torch.zeros(4))
    assert calls == [("warmup", 1, False, 0.999)]


def test_error_word_is_checked_every_n_compressed_steps_and_raises(calls):
    o = opt.OneBitAdam(torch.zeros(4), freeze_step=1, check_every=2)
    for _ in range(5):
        o.step(torch.zeros(4))
    assert [c[0] for c in calls] == ["warmup", "compress", "compress", "status", "compress", "compress", "status"]
    calls.clear()
    o.workspace[0] = 2                     # a wait gave up
    o.step(torch.zeros(4))
    assert calls == [("compress", [0, 4], 0.9, 1e-3)]
    with pytest.raises(opt.WaitTimeout):
        o.step(torch.zeros(4))
    assert [c[0] for c in calls][-2:] == ["status", "init"]
    assert int(o.workspace[0]) == 0
    calls.clear()
    never = opt.OneBitAdam(torch.zeros(4), freeze_step=0, check_every=0)
    never.workspace[0] = 1
    never.step(torch.zeros(4))
    assert calls == [("compress", [0, 4], 0.9, 1e-3)]


@pytest.fixture
def wcalls(monkeypatch):
    """Recorders for the W-worker driver's library calls."""
    log = []
    monkeypatch.setattr(ob, "onebit_plan_create", lambda co, to=None, tk=None: ("plan", np.asarray(co).tolist()))
    monkeypatch.setattr(ob, "onebit_plan_words", lambda p: 3)
    monkeypatch.setattr(ob, "onebit_plan_chunks", lambda p: 2)
    monkeypatch.setattr(ob, "onebit_plan_workspace_bytes", lambda p: 64)
    monkeypatch.setattr(ob, "onebit_average_rows", lambda g, out, stream=None: log.append(("average", g.shape[0])))
    monkeypatch.setattr(ob, "onebit_adam_warmup_step", lambda x, m, v, g, **k: log.append(("warmup", k["step"])))

    def comp(plan, g, m, e, v, x, xb, bits, scales, **k):
        assert v is None and x is None and xb is None and k["lr"] == 0.0
        log.append(("worker", "fp32"))

    def comp_packed(plan, g, mb, ms, e, v, x, xb, bits, scales, **k):
        assert v is None and x is None and xb is None
        log.append(("worker", "packed", id(mb)))

    def server(plan, wb, ws, es, sb, ss, m_out, wsp, stream=None):
        log.append(("server", m_out is not None, id(sb)))

    monkeypatch.setattr(ob, "onebit_compress_update", comp)
    monkeypatch.setattr(ob, "onebit_compress_update_packed", comp_packed)
    monkeypatch.setattr(ob, "onebit_server_reduce", server)
    monkeypatch.setattr(ob, "onebit_momentum_update", lambda m, mask, v, x, xb, **k: log.append(("finish", "fp32")))
    monkeypatch.setattr(ob, "onebit_momentum_update_packed",
                        lambda plan, mb, ms, mask, v, x, xb, **k: log.append(("finish", "packed", id(mb))))
    monkeypatch.setattr(ob, "onebit_workspace_status", lambda ws, stream=None: log.append(("status",)) or 0)
    monkeypatch.setattr(ob, "onebit_decompress", lambda plan, b, s, mask, out, stream=None: log.append(("decompress",)))
    return log


def test_workers_phases_and_call_sequence(wcalls):
    o = opt.OneBitAdamWorkers(torch.zeros(10), 3, chunk_offsets=[0, 4, 10], freeze_step=2)
    g = o.gradient_buffer()
    for _ in range(4):
        o.step(g)
    kinds = [c[0] for c in wcalls]
    assert kinds == ["average", "warmup", "average", "warmup",
                     "worker", "worker", "worker", "server", "finish", "status",
                     "worker", "worker", "worker", "server", "finish", "status"]
    assert all(c[1] == "fp32" for c in wcalls if c[0] in ("worker", "finish"))
    assert all(c[1] is True for c in wcalls if c[0] == "server")          # m_out written
    assert o.worker_error.shape == (3, 10) and o.server_error.shape == (10,)
    with pytest.raises(ValueError):
        o.step(torch.zeros(2, 10))


def test_workers_packed_momentum_alternates_pairs_and_checkpoint_resets_errors(wcalls):
    o = opt.OneBitAdamWorkers(torch.zeros(8), 2, freeze_step=0, packed_momentum=True,
                              exp_avg_mask=torch.ones(8, dtype=torch.bool))
    g = o.gradient_buffer()
    for _ in range(3):
        o.step(g)
    steps = [c for c in wcalls if c[0] != "status"]
    b0, b1 = id(o.server_bits[0]), id(o.server_bits[1])
    # step 1: fp32 momentum, server writes pair 0; step 2: workers read pair 0, server writes 1; step 3: read 1, write 0
    assert steps[:4] == [("worker", "fp32"), ("worker", "fp32"), ("server", True, b0), ("finish", "fp32")]
    assert steps[4:8] == [("worker", "packed", b0), ("worker", "packed", b0), ("server", False, b1),
                          ("finish", "packed", b1)]
    assert steps[8:12] == [("worker", "packed", b1), ("worker", "packed", b1), ("server", False, b0),
                           ("finish", "packed", b0)]
    o.worker_error.fill_(1.0)
    o.server_error.fill_(2.0)
    sd = o.state_dict()
    assert wcalls[-1] == ("decompress",) and set(sd) == {"step", "exp_avg", "exp_avg_sq"}
    o.load_state_dict(sd)
    assert o.current is None and torch.count_nonzero(o.worker_error) == 0 and torch.count_nonzero(o.server_error) == 0
    wcalls.clear()
    o.step(g)
    assert wcalls[0] == ("worker", "fp32")


def test_workers_rejects_bad_arguments(wcalls):
    with pytest.raises(ValueError):
        opt.OneBitAdamWorkers(torch.zeros(4), 0)
    with pytest.raises(ValueError):
        opt.OneBitAdamWorkers(torch.zeros(4), 2, exp_avg_mask=torch.ones(3, dtype=torch.uint8))
    with pytest.raises(ValueError):
        opt.OneBitAdamWorkers(torch.zeros(4), 2, exp_avg_mask=torch.ones(4, dtype=torch.float32))


def closed_form_variance_steps(freeze, kappa):
    """Update k (0-based) sits at 1 + sum_{j<k} 2^floor(j / kappa); with k = q kappa + r
    that sum is kappa (2^q - 1) + r 2^q."""
    out, k = [], 0
    while True:
        q, r = divmod(k, kappa)
        t = 1 + kappa * (2 ** q - 1) + r * 2 ** q
        if t > freeze:
            return out
        out.append(t)
        k += 1


@pytest.mark.parametrize("freeze,kappa", [(0, 1), (1, 1), (100, 1), (1000, 16), (37, 3), (5000, 7)])
def test_variance_schedule_closed_form(freeze, kappa):
    steps = opt.variance_update_steps(freeze, kappa)
    assert steps == closed_form_variance_steps(freeze, kappa)
    if kappa == 1 and freeze >= 1:
        assert steps == [2 ** i for i in range(freeze.bit_length()) if 2 ** i <= freeze]


def test_zero_one_adam_reduces_to_one_bit_adam_without_doubling(calls):
    o = opt.ZeroOneAdam(torch.zeros(4), var_freeze_step=5, var_update_scaler=10)
    for _ in range(7):
        o.step(torch.zeros(4))
    assert [c[0] for c in calls if c[0] != "status"] == ["warmup"] * 5 + ["compress"] * 2


def test_zero_one_adam_alternates_by_the_schedule(calls):
    o = opt.ZeroOneAdam(torch.zeros(4), var_freeze_step=20, var_update_scaler=2)
    for _ in range(24):
        o.step(torch.zeros(4))
    kinds = [c for c in calls if c[0] in ("warmup", "compress")]
    var_steps = [c[1] for c in kinds if c[0] == "warmup"]
    assert var_steps == [1, 2, 3, 5, 7, 11, 15] == opt.variance_update_steps(20, 2)
    assert len(kinds) == 24
    with pytest.raises(TypeError):
        opt.ZeroOneAdam(torch.zeros(4), freeze_step=3)

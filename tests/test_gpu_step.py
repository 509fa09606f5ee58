"""GPU parity of a full compressed step over W workers held on one GPU, and of the
worker finish after the all-reduce (onebit_momentum_update), against the oracle.

The step follows the DeepSpeed 1-bit Adam guide, sec. 4 (phase two) and sec. 3.5:
every worker forms m1 = b1 m + (1 - b1) g_w from the shared momentum and its own
(fp16) gradient, compresses m1 + e_w with its own error; the server averages the W
streams, adds its error and compresses again; the decompressed server result is
the new momentum, multiplied by the per-element exp_avg_mask; x then takes the
frozen-variance step.  Sizes span several tiles with ragged tails; W = 3 exercises
a divide that is not a power of two.
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, host
from parity import assert_exact, check_bf16, check_scales, check_x, say

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, eps=1e-8, weight_decay=0.01)


def rand_state(n, rng):
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.uniform(0.5, 2.0, n) * 1e-6).astype(np.float32)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    return m, v, x


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4099, (1 << 20) + 3, (9 << 20) + 5])  # the last: several grid passes
@pytest.mark.parametrize("with_mask,x_bf16", [(False, False), (True, False), (False, True), (True, True)])
def test_momentum_update_parity(n, with_mask, x_bf16):
    rng = np.random.default_rng(n + 17)
    m, v, x = rand_state(n, rng)
    mask = (rng.random(n) < 0.6).astype(np.uint8) * rng.integers(1, 256, n).astype(np.uint8) if with_mask else None
    md, vd, xd = (torch.from_numpy(a.copy()).to(DEV) for a in (m, v, x))
    maskd = torch.from_numpy(mask).to(DEV) if with_mask else None
    xbd = torch.zeros(max(n, 1), dtype=torch.bfloat16, device=DEV) if x_bf16 else None
    x_prev = x.copy()
    ob.onebit_momentum_update(md, maskd, vd, xd, xbd, **HP)
    rxb = oracle.momentum_update(m, v, x, mask=mask, want_bf16=x_bf16, **HP)
    torch.cuda.synchronize()
    assert_exact(f"n={n} m", host(md), m)
    check_x(f"n={n} x", host(xd), x, x_prev)
    if x_bf16:
        check_bf16(f"n={n} x_bf16", host(xbd)[:n], rxb)


def test_momentum_update_argument_errors():
    f = lambda k: torch.zeros(k, dtype=torch.float32, device=DEV)  # noqa: E731
    m, v, x = f(64), f(64), f(64)
    mask = torch.ones(80, dtype=torch.uint8, device=DEV)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_momentum_update(m, mask[1:65], v, x, None, **HP)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_momentum_update(m[1:], None, v[1:], x[1:], None, **HP)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_momentum_update(m, None, None, x, None, **HP)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID


def word_base(chunk_off):
    lens = np.diff(chunk_off)
    wb = np.zeros(lens.size + 1, np.int64)
    wb[1:] = np.cumsum((lens + 31) // 32)
    return wb


@pytest.mark.parametrize("workers,grad_dtype,steps", [(3, "f16", 3), (4, "bf16", 3), (1, "f32", 3), (4, "bf16", 20)])
def test_full_step_with_element_mask(workers, grad_dtype, steps):
    """W workers, per-element mask (whole rows of an embedding-like tensor zeroed plus
    scattered elements), x_bf16 copy, 3 steps (20 in the long run); every buffer checked
    after every step, so the worker and server errors never drift from the oracle's."""
    lengths = [5000, 4097, 33, (1 << 14) + 7, 1, 2048 * 3, 65]
    off = W.offsets_from_sizes(lengths)
    n = int(off[-1])
    rng = np.random.default_rng(40 + workers)
    m, v, x = rand_state(n, rng)
    e = (rng.standard_normal((workers, n)) * 1e-5).astype(np.float32)
    es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    mask = np.ones(n, np.uint8)
    rows = mask[off[3]:off[4]][: 128 * 64].reshape(128, 64)
    rows[100:] = 0                                   # rows past the trained length never learn
    mask[rng.random(n) < 0.01] = 0
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    md, vd, xd, esd = (torch.from_numpy(a.copy()).to(DEV) for a in (m, v, x, es))
    npad = (n + 3) // 4 * 4                          # worker rows of e start 16-byte aligned
    ed = torch.zeros((workers, npad), device=DEV)
    ed[:, :n] = torch.from_numpy(e).to(DEV)
    maskd = torch.from_numpy(mask).to(DEV)
    wbits = torch.zeros((workers, words), dtype=torch.int32, device=DEV)
    wscales = torch.zeros((workers, nch), dtype=torch.float32, device=DEV)
    sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sscales = torch.zeros(nch, dtype=torch.float32, device=DEV)
    m_out = torch.zeros(n, device=DEV)
    xbd = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    torch_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[grad_dtype]
    for step in range(steps):
        g32 = [(np.random.default_rng(1000 * step + w).standard_normal(n) * 10.0 ** -(2 + w % 3)).astype(np.float32)
               for w in range(workers)]
        gd = [torch.from_numpy(g).to(DEV).to(torch_dt) for g in g32]
        gh = [host(t) if grad_dtype == "bf16" else t.cpu().numpy() for t in gd]
        # GPU step
        for w in range(workers):
            ob.onebit_compress_update(plan, gd[w], md, ed[w, :n], None, None, None, wbits[w], wscales[w], lr=0.0,
                                      beta1=0.9, eps=1e-8, weight_decay=0.0, workspace=ws)
        ob.onebit_server_reduce(plan, wbits, wscales, esd, sbits, sscales, m_out, ws)
        ob.onebit_momentum_update(m_out, maskd, vd, xd, xbd, **HP)
        md.copy_(m_out)
        # oracle step
        rb, rs = [], []
        for w in range(workers):
            b, s, _ = oracle.compress_update(off, gh[w], m, e[w], beta1=0.9)
            rb.append(b)
            rs.append(s)
        sb, ss, mo = oracle.server_reduce(off, np.stack(rb), np.stack(rs), es)
        x_prev = x.copy()
        rxb = oracle.momentum_update(mo, v, x, mask=mask, want_bf16=True, **HP)
        m = mo
        torch.cuda.synchronize()
        tag = f"W={workers} {grad_dtype} step {step}"
        for w in range(workers):
            assert_exact(f"{tag} worker {w} bits", host(wbits[w]).view(np.uint32), rb[w])
            assert check_scales(f"{tag} worker {w} scales", host(wscales[w]), rs[w]) == 0
            assert_exact(f"{tag} worker {w} e", host(ed[w, :n]), e[w])
        assert_exact(f"{tag} server bits", host(sbits).view(np.uint32), sb)
        assert check_scales(f"{tag} server scales", host(sscales), ss) == 0
        assert_exact(f"{tag} server e", host(esd), es)
        assert_exact(f"{tag} m", host(md), m)
        assert np.all(host(md)[mask == 0] == 0)
        check_x(f"{tag} x", host(xd), x, x_prev)
        check_bf16(f"{tag} x_bf16", host(xbd), rxb)
        say(f"  {tag}: all buffers match")
    assert ob.onebit_workspace_status(ws) == 0

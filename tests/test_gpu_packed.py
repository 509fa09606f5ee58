"""GPU parity of the packed-momentum calls (onebit_compress_update_packed,
onebit_momentum_update_packed): the momentum held as the previous step's sign words
and chunk scales.

From a common state, one fp32-momentum step is taken; then for three steps the
fp32 path (onebit_compress_update) and the packed path run side by side on copies
of the state.  Every step the two must agree bit for bit (bits, scales, e, x and
the bf16 copy), the fp32 path's m must equal the masked decompression of the packed
path's words, and the packed path must match the oracle run with m taken as that
decompression.  Cases: edge chunk lengths (empty, 1, 31-33, ragged tails,
2^20 + 5), masked tensors sharing chunks and tiles, a two-pass chunk next to
one-pass chunks, fp32 / bf16 / fp16 gradients, full-size BERT-Large vector.  The
W-worker step (packed compress-only workers with an element mask, server, packed
finish) must reproduce the fp32-momentum W-worker step bit for bit in every buffer.
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, H, host
from parity import assert_exact, check_bf16, check_x, say

pytestmark = pytest.mark.gpu


def masked_elements(n, tensor_off, keep):
    mk = np.zeros(n, bool)
    if tensor_off is not None:
        for t in range(len(keep)):
            if not keep[t]:
                mk[tensor_off[t]:tensor_off[t + 1]] = True
    return mk


def to_dev_grad(g, dt):
    t = torch.from_numpy(g).to(DEV)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
        return t, host(t)
    if dt == "f16":
        t = t.to(torch.float16)
        return t, t.cpu().numpy()
    return t, g


def run(chunk_off, tensor_off=None, keep=None, steps=3, dt="f32", x_bf16=False, seed=0, h=None):
    hp = dict(H)
    hp.update(h or {})
    off = np.asarray(chunk_off, np.int64)
    n = int(off[-1])
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = np.zeros(n, np.float32)
    v = (rng.uniform(0.5, 2, n) * 1e-6).astype(np.float32)
    mk = masked_elements(n, tensor_off, keep)
    plan = ob.onebit_plan_create(off, tensor_off, keep)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    nb = lambda: torch.zeros(max(words, 1), dtype=torch.int32, device=DEV)  # noqa: E731
    ns = lambda: torch.zeros(max(nch, 1), dtype=torch.float32, device=DEV)  # noqa: E731
    # state A (fp32 m) and state B (packed m)
    xa, ma, ea, va = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, e, v))
    xbA = torch.zeros(max(n, 1), dtype=torch.bfloat16, device=DEV) if x_bf16 else None
    xbB = torch.zeros(max(n, 1), dtype=torch.bfloat16, device=DEV) if x_bf16 else None
    bitsA, scA = nb(), ns()
    g0 = (np.random.default_rng(seed + 1).standard_normal(n) * 1e-3).astype(np.float32)
    gd, _ = to_dev_grad(g0, dt)
    ob.onebit_compress_update(plan, gd, ma, ea, va, xa, xbA, bitsA, scA, workspace=ws, **hp)
    xb_, eb_ = xa.clone(), ea.clone()
    pb = [bitsA.clone(), nb()]      # packed path: ping-pong words and scales
    ps = [scA.clone(), ns()]
    xr, er = host(xa), host(ea)     # oracle state follows the packed path
    for step in range(steps):
        g = (np.random.default_rng(seed + 10 + step).standard_normal(n) * 1e-3).astype(np.float32)
        gd, gh = to_dev_grad(g, dt)
        cur, nxt = step % 2, (step + 1) % 2
        m_in = oracle.decompress(off, host(pb[cur]).view(np.uint32)[:words], host(ps[cur])[:nch]) if n else m[:0]
        m_in = np.where(mk, np.float32(0), m_in).astype(np.float32)
        ob.onebit_compress_update(plan, gd, ma, ea, va, xa, xbA, bitsA, scA, workspace=ws, **hp)
        ob.onebit_compress_update_packed(plan, gd, pb[cur], ps[cur], eb_, va, xb_, xbB, pb[nxt], ps[nxt],
                                         workspace=ws, **hp)
        x_prev = xr.copy()
        rb, rs, rxb = oracle.compress_update(off, gh, m_in, er, v, xr, tensor_off=tensor_off, tensor_keep=keep,
                                             want_bf16=x_bf16, **hp)
        torch.cuda.synchronize()
        tag = f"{dt} step {step}"
        assert_exact(f"{tag} bits A/B", host(pb[nxt])[:words], host(bitsA)[:words])
        assert_exact(f"{tag} scales A/B", host(ps[nxt])[:nch], host(scA)[:nch])
        assert_exact(f"{tag} e A/B", host(eb_), host(ea))
        assert_exact(f"{tag} x A/B", host(xb_), host(xa))
        if x_bf16:
            assert_exact(f"{tag} x_bf16 A/B", host(xbB), host(xbA))
        m_packed = oracle.decompress(off, host(pb[nxt]).view(np.uint32)[:words], host(ps[nxt])[:nch]) if n else m[:0]
        assert_exact(f"{tag} fp32 m = masked decompression", host(ma), np.where(mk, np.float32(0), m_packed))
        assert_exact(f"{tag} bits vs oracle", host(pb[nxt]).view(np.uint32)[:words], rb)
        assert_exact(f"{tag} scales vs oracle", host(ps[nxt])[:nch], rs)
        assert_exact(f"{tag} e vs oracle", host(eb_), er)
        check_x(f"{tag} x vs oracle", host(xb_), xr, x_prev)
        if x_bf16:
            check_bf16(f"{tag} x_bf16 vs oracle", host(xbB)[:n], rxb)
        xr = host(xb_)            # follow the device's x exactly (x is toleranced, not bit-pinned)
    assert ob.onebit_workspace_status(ws) == 0
    say(f"  packed momentum {dt}: {steps} steps match")


LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 4095, 4097, 1 << 20, (1 << 20) + 5, 0, 7, 8192, 12]


@pytest.mark.parametrize("dt,x_bf16", [("f32", False), ("bf16", True), ("f16", False)])
def test_packed_edge_lengths(dt, x_bf16):
    run(W.offsets_from_sizes(LENGTHS), dt=dt, x_bf16=x_bf16, seed=31)


def test_packed_masks_sharing_chunks():
    t_off = W.offsets_from_sizes([100, 37, 5000, 64, 9000, 4096, 4096, 11])
    keep = np.array([1, 0, 1, 0, 1, 0, 0, 1], np.uint8)
    c_off = W.offsets_from_sizes([120, 8195, 1000, 12000, 1089])
    run(c_off, t_off, keep, x_bf16=True, seed=32, h=dict(weight_decay=0.01))


def test_packed_two_pass_chunk():
    big = max(ob.onebit_onepass_max_elements(), 1) + 4097
    run(W.offsets_from_sizes([5000, big, 3, 70001]), steps=2, seed=33)


def test_packed_full_size_bert_large():
    wl = W.bert_like()
    hp = dict(lr=wl.hyper["lr"], beta1=wl.hyper["beta1"], eps=wl.hyper["eps"], weight_decay=wl.hyper["weight_decay"])
    x, m, e, v = W.init_state(wl, device=DEV)
    plan = ob.onebit_plan_create(wl.chunk_off, wl.tensor_off, wl.tensor_keep)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    bits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sc = torch.zeros(nch, device=DEV)
    ob.onebit_compress_update(plan, W.gradient(wl, 1, device=DEV), m, e, v, x, None, bits, sc, workspace=ws, **hp)
    pb, ps = [bits.clone(), torch.zeros_like(bits)], [sc.clone(), torch.zeros_like(sc)]
    xb_, eb_ = x.clone(), e.clone()
    for step in range(2):
        g = W.gradient(wl, step + 2, device=DEV)
        cur, nxt = step % 2, (step + 1) % 2
        ob.onebit_compress_update(plan, g, m, e, v, x, None, bits, sc, workspace=ws, **hp)
        ob.onebit_compress_update_packed(plan, g, pb[cur], ps[cur], eb_, v, xb_, None, pb[nxt], ps[nxt],
                                         workspace=ws, **hp)
        torch.cuda.synchronize()
        assert torch.equal(pb[nxt], bits) and torch.equal(ps[nxt], sc)
        assert torch.equal(eb_, e) and torch.equal(xb_, x)
        say(f"  bert_large packed step {step}: bits, scales, e, x identical to the fp32-momentum path")
    assert ob.onebit_workspace_status(ws) == 0


def test_packed_argument_errors():
    off = W.offsets_from_sizes([100])
    plan = ob.onebit_plan_create(off)
    f = torch.zeros(128, device=DEV)
    bits = torch.zeros(8, dtype=torch.int32, device=DEV)
    sc = torch.zeros(4, device=DEV)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    g = f[:100]
    with pytest.raises(ob.OnebitError) as ei:          # words aliasing the output words
        ob.onebit_compress_update_packed(plan, g, bits, sc[1:], f, f, f, None, bits, sc[:1], workspace=ws, **H)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    xb = torch.zeros(128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ob.OnebitError) as ei:          # a bf16 copy of x without an update
        ob.onebit_compress_update_packed(plan, g, bits[4:], sc[1:], f, None, None, xb, bits[:4], sc[:1],
                                         workspace=ws, **H)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError) as ei:          # no scales to decompress
        ob.onebit_compress_update_packed(plan, g, bits[4:], None, f, f, f, None, bits[:4], sc[:1], workspace=ws, **H)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID


@pytest.mark.parametrize("workers,dt", [(3, "f16"), (4, "bf16")])
def test_packed_w_worker_step_with_element_mask(workers, dt):
    """W workers on one GPU with the momentum as the server's words and scales: the
    packed compress-only workers, the server and the packed finish must reproduce the
    fp32-momentum step (compress-only workers, server with m_out, masked finish) bit
    for bit in every buffer, 3 steps after a common first step."""
    lengths = [5000, 4097, 33, (1 << 14) + 7, 1, 2048 * 3, 65]
    off = W.offsets_from_sizes(lengths)
    n = int(off[-1])
    rng = np.random.default_rng(60 + workers)
    hp = dict(lr=1e-3, eps=1e-8, weight_decay=0.01)
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v = torch.from_numpy((rng.uniform(0.5, 2.0, n) * 1e-6).astype(np.float32)).to(DEV)
    mask = np.ones(n, np.uint8)
    mask[rng.random(n) < 0.05] = 0
    maskd = torch.from_numpy(mask).to(DEV)
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    npad = (n + 3) // 4 * 4
    Z = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=DEV)  # noqa: E731
    # path A: fp32 momentum
    mA, eA, esA, xA = Z(n), Z(workers, npad), Z(n), torch.from_numpy(x0.copy()).to(DEV)
    wbA, wsA, sbA, ssA, moA = Z(workers, words, dt=torch.int32), Z(workers, nch), Z(words, dt=torch.int32), Z(nch), Z(n)
    xbA = Z(n, dt=torch.bfloat16)
    # path B: packed momentum (server words / scales ping-pong)
    eB, esB, xB = Z(workers, npad), Z(n), torch.from_numpy(x0.copy()).to(DEV)
    wbB, wsB = Z(workers, words, dt=torch.int32), Z(workers, nch)
    sbB, ssB = [Z(words, dt=torch.int32), Z(words, dt=torch.int32)], [Z(nch), Z(nch)]
    xbB = Z(n, dt=torch.bfloat16)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    h0 = dict(lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0)
    for step in range(4):
        gd = [(torch.from_numpy((np.random.default_rng(900 + 10 * step + w).standard_normal(n) * 1e-3)
                                .astype(np.float32)).to(DEV)).to(tdt) for w in range(workers)]
        # A
        for w in range(workers):
            ob.onebit_compress_update(plan, gd[w], mA, eA[w, :n], None, None, None, wbA[w], wsA[w], workspace=ws, **h0)
        ob.onebit_server_reduce(plan, wbA, wsA, esA, sbA, ssA, moA, ws)
        ob.onebit_momentum_update(moA, maskd, v, xA, xbA, **hp)
        mA.copy_(moA)
        if step == 0:            # B starts from A's state after a common first step
            eB.copy_(eA)
            esB.copy_(esA)
            xB.copy_(xA)
            sbB[0].copy_(sbA)
            ssB[0].copy_(ssA)
            continue
        cur, nxt = (step - 1) % 2, step % 2
        for w in range(workers):
            ob.onebit_compress_update_packed(plan, gd[w], sbB[cur], ssB[cur], eB[w, :n], None, None, None, wbB[w],
                                             wsB[w], workspace=ws, m_mask=maskd, **h0)
        ob.onebit_server_reduce(plan, wbB, wsB, esB, sbB[nxt], ssB[nxt], None, ws)
        ob.onebit_momentum_update_packed(plan, sbB[nxt], ssB[nxt], maskd, v, xB, xbB, **hp)
        torch.cuda.synchronize()
        tag = f"W={workers} {dt} step {step}"
        assert torch.equal(wbB, wbA) and torch.equal(wsB, wsA), f"{tag}: worker words / scales"
        assert torch.equal(eB, eA), f"{tag}: worker errors"
        assert torch.equal(sbB[nxt], sbA) and torch.equal(ssB[nxt], ssA) and torch.equal(esB, esA), f"{tag}: server"
        assert torch.equal(xB, xA) and torch.equal(xbB, xbA), f"{tag}: x"
        m_dec = oracle.decompress(off, host(sbB[nxt]).view(np.uint32), host(ssB[nxt]))
        assert_exact(f"{tag} fp32 m = masked server decompression", host(mA),
                     np.where(mask == 0, m_dec * np.float32(0), m_dec))
        say(f"  {tag}: packed W-worker step identical to the fp32-momentum step")
    assert ob.onebit_workspace_status(ws) == 0


def test_packed_finish_errors():
    plan = ob.onebit_plan_create(W.offsets_from_sizes([100]))
    f = torch.zeros(128, device=DEV)
    b = torch.zeros(8, dtype=torch.int32, device=DEV)
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_momentum_update_packed(plan, b, None, None, f, f, None, lr=1e-3, eps=1e-8, weight_decay=0.0)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_momentum_update_packed(plan, b, f, None, f[1:], f, None, lr=1e-3, eps=1e-8, weight_decay=0.0)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN

"""GPU parity of onebit_compress_update (and the warmup kernel) against the oracle.

Sizes span several 4096-element tiles with ragged tails; chunk tables cover the
edge cases of the packing and of the chunk-norm exchange (lengths 0, 1, 2, 31,
32, 33, 63, 64, 65, 4095, 4097, 2^20, 2^20 + 5; starts that are not multiples of
4; all-zero, all-negative, signed-zero and wide-range chunks; masked tensors that
share chunks and tiles with kept ones; a chunk too large to stay resident, which
takes the two-pass path).
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, H, CompressBuffers, host, oracle_compress
from parity import (assert_bits_exact, assert_exact, check_bf16, check_err, check_scales, check_x,
                    per_element, say)

pytestmark = pytest.mark.gpu


def compare(tag, buf, ref_bits, ref_scales, m_gpu, e_gpu, x_gpu, m_ref, e_ref, x_ref, x_prev, xb_ref=None,
            masked=None):
    say(f"  compare {tag}")
    assert_bits_exact(f"{tag} bits", buf.out_bits(), ref_bits)
    nonexact = check_scales(f"{tag} scales", buf.out_scales(), ref_scales)
    sc = per_element(ref_scales, buf.chunk_off)
    if m_gpu is not None:
        check_err(f"{tag} m", m_gpu, m_ref, np.zeros_like(sc))
        if nonexact == 0:
            assert_exact(f"{tag} m", m_gpu, m_ref)
    check_err(f"{tag} e", e_gpu, e_ref, sc)
    if nonexact == 0:
        assert_exact(f"{tag} e", e_gpu, e_ref)
    if x_gpu is not None:
        check_x(f"{tag} x", x_gpu, x_ref, x_prev)
    if masked is not None and masked.any():
        assert np.all(m_gpu[masked] == 0) and np.all(e_gpu[masked] == 0)
    if xb_ref is not None:
        check_bf16(f"{tag} x_bf16", host(buf.xb)[:buf.n], xb_ref)
    assert buf.ws_status() == 0, "a cross-workgroup wait timed out"
    return nonexact


def run_steps(chunk_off, steps, *, init, grads, tensor_off=None, tensor_keep=None, x_bf16=False, bf16_grad=False,
              compress_only=False, h=None):
    """Run `steps` compressed steps on GPU and oracle from the same initial state; each side evolves alone."""
    h = h or {}
    buf = CompressBuffers(chunk_off, tensor_off, tensor_keep, x_bf16=x_bf16)
    x0, m0, e0, v0 = init
    xd, md, ed, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x0, m0, e0, v0))
    xr, mr, er, vr = (a.copy() for a in (x0, m0, e0, v0))
    masked = None
    if tensor_off is not None:
        masked = np.repeat(np.asarray(tensor_keep) == 0, np.diff(tensor_off))
    total_nonexact = 0
    for s in range(steps):
        g = grads(s)
        if g.dtype == np.uint16:      # bf16 bit patterns
            gd = torch.from_numpy(g.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
        else:
            gd = torch.from_numpy(g.copy()).to(DEV)
        x_prev = xr.copy()
        if compress_only:
            buf.step(gd, md, ed, **h)
            rb, rs, _ = oracle_compress(chunk_off, g, mr, er, tensor_off=tensor_off, tensor_keep=tensor_keep, **h)
            torch.cuda.synchronize()
            assert_exact("m untouched", host(md), mr)
            total_nonexact += compare(f"step {s}", buf, rb, rs, None, host(ed), None, None, er, None, None)
        else:
            buf.step(gd, md, ed, vd, xd, **h)
            rb, rs, rxb = oracle_compress(chunk_off, g, mr, er, vr, xr, tensor_off=tensor_off, tensor_keep=tensor_keep,
                                          want_bf16=x_bf16, **h)
            torch.cuda.synchronize()
            total_nonexact += compare(f"step {s}", buf, rb, rs, host(md), host(ed), host(xd), mr, er, xr, x_prev, rxb,
                                      masked)
    return buf, total_nonexact


def rand_state(n, rng, v_scale=1e-6):
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = (rng.uniform(0.5, 2.0, n) * v_scale).astype(np.float32)
    return x, m, e, v


def test_tiny_workload_warmup_then_compressed():
    """1,048,576 fp32 params, one chunk: 5 full-precision Adam steps, freeze v, 5 compressed steps."""
    wl = W.tiny()
    say("tiny workload n=%d" % wl.n)
    x, m, e, v = (t.numpy().copy() for t in W.init_state(wl))
    xd, md, ed, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, e, v))
    buf = CompressBuffers(wl.chunk_off)
    hp = W.HYPER
    for t in range(1, 6):
        g = W.gradient(wl, t).numpy()
        x_prev = x.copy()
        ob.onebit_adam_warmup_step(xd, md, vd, torch.from_numpy(g).to(DEV), lr=hp["lr"], beta1=hp["beta1"],
                                   beta2=hp["beta2"], eps=hp["eps"], weight_decay=hp["weight_decay"],
                                   bias_correction=hp["bias_correction"], step=t)
        oracle.adam_warmup_step(x, m, v, g, lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                weight_decay=hp["weight_decay"], bias_correction=hp["bias_correction"], step=t)
        torch.cuda.synchronize()
        assert_exact(f"warmup {t} m", host(md), m)
        assert_exact(f"warmup {t} v", host(vd), v)
        check_x(f"warmup {t} x", host(xd), x, x_prev)
    for t in range(6, 11):
        g = W.gradient(wl, t).numpy()
        x_prev = x.copy()
        buf.step(torch.from_numpy(g).to(DEV), md, ed, vd, xd)
        rb, rs, _ = oracle_compress(wl.chunk_off, g, m, e, v, x)
        torch.cuda.synchronize()
        n_ne = compare(f"compressed step {t}", buf, rb, rs, host(md), host(ed), host(xd), m, e, x, x_prev)
        assert n_ne == 0, "scale differs from the oracle's"


LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 4095, 4097, 1 << 20, (1 << 20) + 5, 0, 7, 8192, 12]


def edge_state(lengths, rng):
    off = W.offsets_from_sizes(lengths)
    n = int(off[-1])
    x, m, e, v = rand_state(n, rng)
    j = {L: i for i, L in enumerate(lengths)}
    # all-negative chunk; wide dynamic range chunk; zero chunk with signed zeros
    a, b = off[j[4095]], off[j[4095] + 1]
    m[a:b] = -np.abs(m[a:b]) - 1e-3
    a, b = off[j[65]], off[j[65] + 1]
    m[a:b] = (np.float32(10.0) ** np.linspace(-30, 30, b - a)).astype(np.float32) * np.sign(rng.standard_normal(b - a))
    e[a:b] = 0
    a, b = off[j[7]], off[j[7] + 1]
    m[a:b] = SIGNED_ZEROS
    e[a:b] = SIGNED_ZEROS
    return off, (x, m, e, v)


SIGNED_ZEROS = np.array([0, -0.0, 0, -0.0, 0, 0, -0.0], np.float32)   # c = -0 where m, g, e are all -0


@pytest.mark.parametrize("grad_dtype,x_bf16", [("f32", False), ("bf16", True), ("f16", False)])
def test_edge_chunk_lengths(grad_dtype, x_bf16):
    rng = np.random.default_rng(21)
    off, init = edge_state(LENGTHS, rng)
    n = int(off[-1])
    zero_chunk = slice(int(off[13]), int(off[14]))

    def grads(s):
        g = (np.random.default_rng(100 + s).standard_normal(n) * 1e-3).astype(np.float32)
        g[zero_chunk] = SIGNED_ZEROS
        if grad_dtype == "bf16":
            return torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        if grad_dtype == "f16":
            return g.astype(np.float16)
        return g

    say(f"edge lengths grad_dtype={grad_dtype}")
    run_steps(off, 3, init=init, grads=grads, x_bf16=x_bf16)


def test_unaligned_chunk_starts_and_compress_only():
    rng = np.random.default_rng(22)
    off = W.offsets_from_sizes([3, 5, 4097, 1030, 2, 9001, 1])
    n = int(off[-1])
    init = rand_state(n, rng)
    grads = lambda s: (np.random.default_rng(200 + s).standard_normal(n) * 1e-3).astype(np.float32)  # noqa: E731
    say("unaligned starts, update mode")
    run_steps(off, 3, init=init, grads=grads)
    say("unaligned starts, compress-only mode")
    run_steps(off, 3, init=init, grads=grads, compress_only=True)


@pytest.mark.parametrize("grad_dtype,mode", [("f32", "update_xbf16"), ("bf16", "update"), ("f16", "update"),
                                             ("f32", "compress_only"), ("bf16", "compress_only")])
def test_masks_sharing_chunks_and_tiles(grad_dtype, mode):
    rng = np.random.default_rng(23)
    t_off = W.offsets_from_sizes([100, 37, 5000, 64, 9000, 4096, 4096, 11])
    keep = np.array([1, 0, 1, 0, 1, 0, 0, 1], np.uint8)
    c_off = W.offsets_from_sizes([120, 8195, 1000, 12000, 1089])
    n = int(t_off[-1])
    assert int(c_off[-1]) == n
    init = rand_state(n, rng)

    def grads(s):
        g = (np.random.default_rng(300 + s).standard_normal(n) * 1e-3).astype(np.float32)
        if grad_dtype == "bf16":
            return torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return g.astype(np.float16) if grad_dtype == "f16" else g

    say(f"masks sharing chunks, {grad_dtype} gradients, {mode}")
    run_steps(c_off, 3, init=init, grads=grads, tensor_off=t_off, tensor_keep=keep, x_bf16=mode == "update_xbf16",
              compress_only=mode == "compress_only")


def test_weight_decay_and_hyperparameters():
    rng = np.random.default_rng(24)
    off = W.offsets_from_sizes([5000, 70000])
    n = int(off[-1])
    init = rand_state(n, rng)
    grads = lambda s: (np.random.default_rng(400 + s).standard_normal(n) * 1e-3).astype(np.float32)  # noqa: E731
    run_steps(off, 2, init=init, grads=grads, h=dict(lr=3e-4, beta1=0.95, eps=1e-6, weight_decay=0.01))


def test_two_pass_chunk_next_to_one_pass_chunks():
    cap = ob.onebit_device_resident_capacity()
    say(f"device capacity {cap} workgroups, one-pass chunks up to {ob.onebit_onepass_max_elements()}")
    big = max(ob.onebit_onepass_max_elements(), 1) + 4097
    off = W.offsets_from_sizes([5000, big, 3, 70001])
    buf = CompressBuffers(off)
    st = ob.onebit_plan_stats(buf.plan)
    say(f"plan stats {st}")
    assert st["twopass_tiles"] > 0 and (cap == 0 or st["onepass_tiles"] > 0)
    n = int(off[-1])
    rng = np.random.default_rng(25)
    init = rand_state(n, rng)
    grads = lambda s: (np.random.default_rng(500 + s).standard_normal(n) * 1e-3).astype(np.float32)  # noqa: E731
    run_steps(off, 2, init=init, grads=grads)
    run_steps(off, 2, init=init, grads=grads, compress_only=True)


def test_bert_small_three_steps():
    wl = W.bert_small()
    init = tuple(t.numpy().copy() for t in W.init_state(wl))
    grads = lambda s: W.gradient(wl, s + 1).numpy()  # noqa: E731
    say(f"bert_small n={wl.n} chunks={wl.n_chunks}")
    run_steps(wl.chunk_off, 3, init=init, grads=grads, tensor_off=wl.tensor_off, tensor_keep=wl.tensor_keep)


def test_forty_steps_with_masks_no_drift():
    """40 compressed steps over a mixed chunk table (one-pass chunks of many lengths,
    masked tensors sharing chunks with kept ones, bf16 copy of x), fresh gradients of
    changing scale each step; after every step bits, scales, m and e equal the oracle's
    and x is within tolerance, so nothing drifts as e and m evolve."""
    lengths = [1, 33, 4097, 65541, 1000, 131072, 7, 70000, 64, 2048 * 5 + 3]
    c_off = W.offsets_from_sizes(lengths)
    n = int(c_off[-1])
    t_off = np.array([0, 20, 4131, 60000, 140000, 201113, 270000, n], np.int64)
    keep = np.array([1, 0, 1, 1, 0, 1, 1], np.uint8)
    rng = np.random.default_rng(4040)
    init = rand_state(n, rng)
    scale = 10.0 ** rng.uniform(-4, -2, len(lengths))
    per = np.repeat(scale, np.diff(c_off))

    def grads(s):
        g = np.random.default_rng(9000 + s).standard_normal(n) * per * (1.0 + 0.5 * np.sin(s))
        g[np.repeat(keep == 0, np.diff(t_off))] = 0.0
        return g.astype(np.float32)
    say(f"forty steps n={n}")
    _, nonexact = run_steps(c_off, 40, init=init, grads=grads, tensor_off=t_off, tensor_keep=keep, x_bf16=True)
    assert nonexact == 0


def test_repeat_is_bit_identical_and_workspace_shared_across_plans():
    rng = np.random.default_rng(26)
    offs = [W.offsets_from_sizes([70000, 4097, 1 << 20]), W.offsets_from_sizes([33, 9000])]
    ws = None
    for off in offs:
        n = int(off[-1])
        x, m, e, v = rand_state(n, rng)
        g = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).to(DEV)
        outs = []
        for rep in range(2):
            buf = CompressBuffers(off, workspace=ws)
            ws = buf.ws if ws is None else ws
            xd, md, ed, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, e, v))
            buf.step(g, md, ed, vd, xd)
            torch.cuda.synchronize()
            outs.append([host(t) for t in (md, ed, xd)] + [buf.out_bits(), buf.out_scales()])
            assert buf.ws_status() == 0
        for a, b in zip(*outs):
            assert_exact("repeat", a, b)


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_warmup_kernel_several_grid_passes(gdt):
    """13 * 2^20 + 5 elements: more than one pass of the grid-stride loop (at most
    six workgroups per CU x 4096 elements each per pass), plus a ragged tail."""
    n = (13 << 20) + 5
    rng = np.random.default_rng(5)
    x, m, _, v = rand_state(n, rng)
    xd, md, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, v))
    for t in range(1, 3):
        g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        gt = torch.from_numpy(g32).to(DEV)
        if gdt == "bf16":
            gt = gt.to(torch.bfloat16)
            g = host(gt)
        else:
            g = g32
        hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, bias_correction=True, step=t)
        say(f"warmup n={n} {gdt} step {t}")
        x_prev = x.copy()
        ob.onebit_adam_warmup_step(xd, md, vd, gt, **hp)
        oracle.adam_warmup_step(x, m, v, g, **hp)
        torch.cuda.synchronize()
        assert_exact(f"n={n} m", host(md), m)
        assert_exact(f"n={n} v", host(vd), v)
        check_x(f"n={n} x", host(xd), x, x_prev)


def test_warmup_kernel_edge_sizes():
    for n in (1, 3, 4, 5, 4099, (1 << 20) + 3):
        for gdt in ("f32", "bf16", "f16"):
            for bias, wd in ((False, 0.0), (True, 0.01)):
                rng = np.random.default_rng(n)
                x, m, _, v = rand_state(n, rng)
                xd, md, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, v))
                for t in range(1, 4):
                    g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
                    gt = torch.from_numpy(g32).to(DEV)
                    if gdt == "bf16":
                        gt = gt.to(torch.bfloat16)
                        g = host(gt)
                    elif gdt == "f16":
                        gt = gt.to(torch.float16)
                        g = gt.cpu().numpy()
                    else:
                        g = g32
                    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, bias_correction=bias, step=t)
                    x_prev = x.copy()
                    ob.onebit_adam_warmup_step(xd, md, vd, gt, **hp)
                    oracle.adam_warmup_step(x, m, v, g, **hp)
                    torch.cuda.synchronize()
                    assert_exact(f"n={n} m", host(md), m)
                    assert_exact(f"n={n} v", host(vd), v)
                    check_x(f"n={n} x", host(xd), x, x_prev)


def test_argument_errors():
    buf = CompressBuffers(W.offsets_from_sizes([100]))
    n = 100
    f = lambda: torch.zeros(n, dtype=torch.float32, device=DEV)  # noqa: E731
    g, m, e, v, x = f(), f(), f(), f(), f()
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_update(buf.plan, g, m, e, v, None, None, buf.bits, buf.scales, workspace=buf.ws, **H)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError) as ei:
        ob.onebit_compress_update(buf.plan, g[1:], m, e, v, x, None, buf.bits, buf.scales, workspace=buf.ws, **H)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN
    with pytest.raises(ob.OnebitError) as ei:   # W = 0 workers
        ob.onebit_server_reduce(buf.plan, buf.bits.view(1, -1), torch.zeros((0, 1), device=DEV), e, buf.bits,
                                buf.scales, None, buf.ws)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID

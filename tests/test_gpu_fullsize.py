"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times, on sampled chunks / buckets that the oracle recomputes one by one.

  bert_large  335,143,938 fp32 params, 393 chunks (one per tensor), 8 masked, 3 steps
  gpt2_xl     1,557,611,200 params, bf16 gradients, 2^20 chunks, bf16 copy of x, 3 steps
  allreduce   16 workers x 64M fp32, 16 chunks of 4M, server stage, 3 steps
  qsdp        1.3e9 bf16 weights, buckets of 1024, 4- and 8-bit codes

Each step copies the sampled chunks' inputs to the host before the GPU step,
runs the oracle on exactly those chunks, and compares bit for bit (bits, scales,
m, e; codes, bucket min/max) or within the stated tolerance (x, bf16 copy).
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, H, host
from parity import assert_exact, check_bf16, check_scales, check_x, local_tensor_table, say

pytestmark = pytest.mark.gpu


def word_base(chunk_off):
    lens = np.diff(chunk_off)
    wb = np.zeros(lens.size + 1, np.int64)
    wb[1:] = np.cumsum((lens + 31) // 32)
    return wb


def run_sampled(wl, sample, steps=3):
    x, m, e, v = W.init_state(wl, device=DEV)
    plan = ob.onebit_plan_create(wl.chunk_off, wl.tensor_off, wl.tensor_keep)
    say(f"{wl.name}: n={wl.n} chunks={wl.n_chunks} plan {ob.onebit_plan_stats(plan)}")
    bits = torch.zeros(ob.onebit_plan_words(plan), dtype=torch.int32, device=DEV)
    scales = torch.zeros(wl.n_chunks, dtype=torch.float32, device=DEV)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    xb = torch.zeros(wl.n, dtype=torch.bfloat16, device=DEV) if wl.x_bf16_copy else None
    wb = word_base(wl.chunk_off)
    hp = dict(lr=wl.hyper["lr"], beta1=wl.hyper["beta1"], eps=wl.hyper["eps"], weight_decay=wl.hyper["weight_decay"])
    for step in range(1, steps + 1):
        g = W.gradient(wl, step, device=DEV)
        before = {}
        for j in sample:
            lo, hi = int(wl.chunk_off[j]), int(wl.chunk_off[j + 1])
            before[j] = [host(t[lo:hi]) for t in (g, m, e, v, x)]
        ob.onebit_compress_update(plan, g, m, e, v, x, xb, bits, scales, workspace=ws, **hp)
        torch.cuda.synchronize()
        gs = host(scales)
        for j in sample:
            lo, hi = int(wl.chunk_off[j]), int(wl.chunk_off[j + 1])
            gj, mj, ej, vj, xj = before[j]
            x_prev = xj.copy()
            to, tk = local_tensor_table(wl.tensor_off, wl.tensor_keep, lo, hi)
            rb, rs, rxb = oracle.compress_update(np.array([0, hi - lo], np.int64), gj, mj, ej, vj, xj,
                                                 tensor_off=to, tensor_keep=tk, want_bf16=wl.x_bf16_copy, **hp)
            tag = f"{wl.name} step {step} chunk {j} [{lo},{hi})"
            assert_exact(f"{tag} bits", host(bits[wb[j]:wb[j + 1]]).view(np.uint32), rb)
            nonexact = check_scales(f"{tag} scale", gs[j:j + 1], rs)
            if nonexact == 0:
                assert_exact(f"{tag} m", host(m[lo:hi]), mj)
                assert_exact(f"{tag} e", host(e[lo:hi]), ej)
            check_x(f"{tag} x", host(x[lo:hi]), xj, x_prev)
            if xb is not None:
                check_bf16(f"{tag} x_bf16", host(xb[lo:hi]), rxb)
        say(f"  step {step}: {len(sample)} chunks match")
    assert ob.onebit_workspace_status(ws) == 0


def test_bert_large_full_size():
    wl = W.bert_like()
    lens = np.diff(wl.chunk_off)
    masked = list(np.nonzero(wl.tensor_keep == 0)[0])
    pick = {0, 1, wl.n_chunks - 1, int(np.argmax(lens)), int(np.nonzero(lens == 4 << 20)[0][0]),
            int(np.nonzero(lens == 1 << 20)[0][0]), int(np.nonzero(lens == 1024)[0][-1])}
    pick |= set(int(j) for j in masked)
    pick |= set(int(j) for j in np.random.default_rng(1).choice(wl.n_chunks, 6, replace=False))
    run_sampled(wl, sorted(pick))


def test_gpt2_xl_full_size():
    wl = W.gpt2_like()
    pick = {0, wl.n_chunks - 1, wl.n_chunks - 2} | set(
        int(j) for j in np.random.default_rng(2).choice(wl.n_chunks, 5, replace=False))
    run_sampled(wl, sorted(pick))


def test_simulated_allreduce_full_size():
    a = W.AllreduceWorkload()
    off = a.chunk_off
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    wb = word_base(off)
    say(f"allreduce W={a.W} n={a.n} chunks={nch} plan {ob.onebit_plan_stats(plan)}")
    m = torch.zeros(a.n, device=DEV)
    e = torch.zeros((a.W, a.n), device=DEV)
    es = torch.zeros(a.n, device=DEV)
    wbits = torch.zeros((a.W, words), dtype=torch.int32, device=DEV)
    wscales = torch.zeros((a.W, nch), dtype=torch.float32, device=DEV)
    sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sscales = torch.zeros(nch, dtype=torch.float32, device=DEV)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    hp = dict(lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0)
    for step in range(1, a.steps + 1):
        sample = sorted(set(int(j) for j in np.random.default_rng(step).choice(nch, 2, replace=False)) | {nch - 1})
        grads = [W.allreduce_gradient(a, step, w, device=DEV) for w in range(a.W)]
        before = {j: (host(m[off[j]:off[j + 1]]), [host(e[w, off[j]:off[j + 1]]) for w in range(a.W)],
                      [host(gw[off[j]:off[j + 1]]) for gw in grads], host(es[off[j]:off[j + 1]])) for j in sample}
        for w in range(a.W):
            ob.onebit_compress_update(plan, grads[w], m, e[w], None, None, None, wbits[w], wscales[w], workspace=ws,
                                      **hp)
        ob.onebit_server_reduce(plan, wbits, wscales, es, sbits, sscales, m, ws)
        torch.cuda.synchronize()
        for j in sample:
            lo, hi = int(off[j]), int(off[j + 1])
            mj, ejs, gjs, esj = before[j]
            loc = np.array([0, hi - lo], np.int64)
            rbits, rsc = [], []
            for w in range(a.W):
                rb, rs, _ = oracle.compress_update(loc, gjs[w], mj, ejs[w], **hp)
                assert_exact(f"step {step} chunk {j} worker {w} bits",
                             host(wbits[w, wb[j]:wb[j + 1]]).view(np.uint32), rb)
                assert check_scales(f"worker {w} scale", host(wscales[w, j:j + 1]), rs) == 0
                assert_exact(f"step {step} chunk {j} worker {w} e", host(e[w, lo:hi]), ejs[w])
                rbits.append(rb)
                rsc.append(rs)
            sb, ss, m_out = oracle.server_reduce(loc, np.stack(rbits), np.stack(rsc), esj)
            assert_exact(f"step {step} chunk {j} server bits", host(sbits[wb[j]:wb[j + 1]]).view(np.uint32), sb)
            assert check_scales("server scale", host(sscales[j:j + 1]), ss) == 0
            assert_exact(f"step {step} chunk {j} server e", host(es[lo:hi]), esj)
            assert_exact(f"step {step} chunk {j} m", host(m[lo:hi]), m_out)
        say(f"  step {step}: chunks {sample} match")
        del grads
    assert ob.onebit_workspace_status(ws) == 0


@pytest.mark.parametrize("bits", [4, 8])
def test_qsdp_full_size(bits):
    q = W.QsdpWorkload()
    xq = W.qsdp_weights(q, device=DEV)
    nb = (q.n + q.bucket - 1) // q.bucket
    nbytes = (q.n + 1) // 2 if bits == 4 else q.n
    codes = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    bmin = torch.zeros(nb, device=DEV)
    bmax = torch.zeros(nb, device=DEV)
    y16 = torch.zeros(q.n, dtype=torch.bfloat16, device=DEV)
    per = 2 if bits == 4 else 1
    for seed in (0, 63):
        ob.qsdp_quantize(xq, q.bucket, bits, seed, codes, bmin, bmax)
        ob.qsdp_dequantize(codes, bmin, bmax, q.n, q.bucket, bits, y16)
        torch.cuda.synchronize()
        sample = sorted({0, nb - 1, nb - 2} | set(int(b) for b in np.random.default_rng(seed).choice(nb, 61, replace=False)))
        for b in sample:
            lo, hi = b * q.bucket, min((b + 1) * q.bucket, q.n)
            xs = host(xq[lo:hi])
            rc, rmn, rmx = oracle.qsdp_quantize(xs, bucket=q.bucket, bits=bits, seed=seed, first_index=lo)
            assert_exact(f"seed {seed} bucket {b} codes", host(codes[lo // per:(hi + per - 1) // per]), rc)
            assert_exact(f"seed {seed} bucket {b} min", host(bmin[b:b + 1]), rmn)
            assert_exact(f"seed {seed} bucket {b} max", host(bmax[b:b + 1]), rmx)
            r16, _ = oracle.qsdp_dequantize(rc, rmn, rmx, hi - lo, bucket=q.bucket, bits=bits)
            assert_exact(f"seed {seed} bucket {b} y", host(y16[lo:hi]), r16)
        say(f"  qsdp bits={bits} seed={seed}: {len(sample)} buckets match")

"""Edge cases of the boundary on the GPU: empty inputs for every entry point, the
largest worker count the server stage accepts (1024, with random pad bits in the
workers' last words) and the first one it rejects."""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, H, host
from parity import assert_exact, check_scales, say

pytestmark = pytest.mark.gpu


def test_empty_inputs_are_no_ops():
    z = torch.zeros(0, device=DEV)
    zb = torch.zeros(0, dtype=torch.bfloat16, device=DEV)
    z8 = torch.zeros(16, dtype=torch.uint8, device=DEV)
    z4 = torch.zeros(4, device=DEV)
    ob.onebit_adam_warmup_step(z, z, z, z, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                               bias_correction=True, step=1)
    ob.onebit_momentum_update(z, None, z, z, None, lr=1e-3, eps=1e-8, weight_decay=0.0)
    ob.qsdp_quantize(zb, 1024, 4, 0, z8, z4, z4)
    ob.qsdp_dequantize(z8, z4, z4, 0, 1024, 4, zb)
    ob.qsgd_quantize(zb, 1024, 4, 0, z8, z4)
    ob.qsgd_reduce(z8, z4, 0, 1024, 4, out_f32=z)
    ob.loco_quantize(zb, z, 1024, 8, 0.5, 0, z8, z4)
    # a plan over empty chunks: no words, scale 0 for each chunk
    plan = ob.onebit_plan_create(np.array([0, 0, 0], np.int64))
    assert ob.onebit_plan_elements(plan) == 0 and ob.onebit_plan_words(plan) == 0
    scales = torch.full((2,), 7.0, device=DEV)
    bits = torch.zeros(4, dtype=torch.int32, device=DEV)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    ob.onebit_compress_update(plan, z, z, z, z, z, None, bits, scales, workspace=ws, **H)
    ob.onebit_server_reduce(plan, bits.view(1, -1), scales.view(1, -1), z, bits, scales, None, ws)
    torch.cuda.synchronize()
    assert np.all(host(scales) == 0)
    assert ob.onebit_workspace_status(ws) == 0


def test_server_at_the_worker_limit():
    off = W.offsets_from_sizes([33, 4097, 900])
    n = int(off[-1])
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    Wn = 1024
    rng = np.random.default_rng(1024)
    wbits = rng.integers(0, 2 ** 32, size=(Wn, words), dtype=np.uint64).astype(np.uint32)   # pad bits random too
    wscales = (rng.uniform(0.5, 2.0, (Wn, nch)) * 10.0 ** rng.uniform(-5, -2, (Wn, 1))).astype(np.float32)
    es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    esd = torch.from_numpy(es.copy()).to(DEV)
    sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sscales = torch.zeros(nch, device=DEV)
    m_out = torch.zeros(n, device=DEV)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    wb = torch.from_numpy(wbits.view(np.int32)).to(DEV)
    wsc = torch.from_numpy(wscales).to(DEV)
    ob.onebit_server_reduce(plan, wb, wsc, esd, sbits, sscales, m_out, ws)
    rb, rs, rm = oracle.server_reduce(off, wbits, wscales, es)
    torch.cuda.synchronize()
    assert_exact("server bits", host(sbits).view(np.uint32), rb)
    assert check_scales("server scales", host(sscales), rs) == 0
    assert_exact("server e", host(esd), es)
    assert_exact("server m", host(m_out), rm)
    assert ob.onebit_workspace_status(ws) == 0
    say(f"  W={Wn}: server stage matches")
    with pytest.raises(ob.OnebitError) as ei:
        more = torch.zeros((Wn + 1, words), dtype=torch.int32, device=DEV)
        ob.onebit_server_reduce(plan, more, torch.zeros((Wn + 1, nch), device=DEV), esd, sbits, sscales, None, ws)
    assert ei.value.status == ob.ONEBIT_ERR_INVALID


def test_forced_wait_timeouts_are_reported_and_recoverable():
    """With a spin limit of one re-poll, cross-workgroup waits on large chunks give up:
    the call still completes, the workspace reports the failure, and after
    onebit_workspace_init and the default limit the same step matches the oracle.
    (Should every wait happen to succeed, the results must already match.)"""
    off = W.fixed_chunks(16 << 20, 4 << 20)
    n = int(off[-1])
    rng = np.random.default_rng(77)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e0 = np.zeros(n, np.float32)
    plan = ob.onebit_plan_create(off)
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
    bits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sc = torch.zeros(nch, device=DEV)
    gd = torch.from_numpy(g).to(DEV)
    er = e0.copy()
    rb, rs, _ = oracle.compress_update(off, g, m0.copy(), er, **H)
    try:
        ob.onebit_set_spin_limit(1)
        md, ed = torch.from_numpy(m0.copy()).to(DEV), torch.from_numpy(e0.copy()).to(DEV)
        ob.onebit_compress_update(plan, gd, md, ed, None, None, None, bits, sc, workspace=ws, **H)
        torch.cuda.synchronize()
        status = ob.onebit_workspace_status(ws)
    finally:
        ob.onebit_set_spin_limit(0)
    say(f"  spin limit 1: workspace status {status}")
    if status == 0:
        assert_exact("bits with every wait satisfied", host(bits).view(np.uint32), rb)
    else:
        assert status in (1, 2)
    ob.onebit_workspace_init(ws)
    md, ed = torch.from_numpy(m0.copy()).to(DEV), torch.from_numpy(e0.copy()).to(DEV)
    ob.onebit_compress_update(plan, gd, md, ed, None, None, None, bits, sc, workspace=ws, **H)
    torch.cuda.synchronize()
    assert ob.onebit_workspace_status(ws) == 0
    assert_exact("bits after re-initialization", host(bits).view(np.uint32), rb)
    assert check_scales("scales after re-initialization", host(sc), rs) == 0
    assert_exact("e after re-initialization", host(ed), er)


def test_library_loaded_before_torch_shares_its_runtime():
    """A fresh process that loads the library before it imports torch: the binding
    brings torch's HIP runtime in first, so plan creation and a warmup step work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import numpy as np\n"
            "from error_compensated_bit_amd import onebit as ob\n"
            "ob.load()\n"
            "p = ob.onebit_plan_create(np.array([0, 4096], np.int64))\n"
            "import torch\n"
            "z = torch.zeros(4096, device='cuda:0')\n"
            "g = torch.ones(4096, device='cuda:0')\n"
            "ob.onebit_adam_warmup_step(z, z.clone(), z.clone(), g, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,"
            " weight_decay=0.0, bias_correction=True, step=1)\n"
            "torch.cuda.synchronize()\n"
            "assert abs(float(z[0]) + 1e-3) < 1e-6, float(z[0])\n"
            "print('ok')\n")
    say("library loaded before torch, fresh process")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]

"""The allocation-free call (onebit_compress_update_static) against the call with a
caller workspace (onebit_compress_update), through the C ABI on the same inputs:
bits, scales, m, e, x and the bf16 copy of x identical bit for bit, over two calls in
a row whose second plan is smaller than the first (the first has a chunk too large
for the one-pass kernel, so both the two-pass and the one-pass launches use the
scratch), with the wait status reported as 0; a compress-only call and a plan with
no chunks; a plan whose workspace would exceed the scratch is refused with
ONEBIT_ERR_NOMEM before anything runs."""
import numpy as np
import pytest
import torch

from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, H, host
from parity import assert_exact, say

pytestmark = pytest.mark.gpu


def state(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = (rng.uniform(0.5, 2.0, n) * 1e-6).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return x, m, e, v, g


def both(off, t_off, keep, seed, update=True, x_bf16=True):
    plan = ob.onebit_plan_create(off, t_off, keep)
    n = int(off[-1])
    words, nch = ob.onebit_plan_words(plan), ob.onebit_plan_chunks(plan)
    x, m, e, v, g = state(n, seed)
    gd = torch.from_numpy(g).to(DEV).to(torch.bfloat16)
    outs = []
    for static in (False, True):
        xd, md, ed, vd = (torch.from_numpy(a.copy()).to(DEV) for a in (x, m, e, v))
        bits = torch.zeros(max(words, 1), dtype=torch.int32, device=DEV)
        scales = torch.zeros(max(nch, 1), device=DEV)
        xb = torch.zeros(max(n, 1), dtype=torch.bfloat16, device=DEV) if (x_bf16 and update) else None
        args = (plan, gd, md, ed, vd if update else None, xd if update else None, xb, bits, scales)
        if static:
            st = torch.full((1,), -1, dtype=torch.int64, device=DEV)
            ob.onebit_compress_update_static(*args, wait_status=st, **H)
        else:
            ws = torch.zeros(ob.onebit_plan_workspace_bytes(plan) // 8, dtype=torch.int64, device=DEV)
            ob.onebit_compress_update(*args, workspace=ws, **H)
        torch.cuda.synchronize()
        outs.append([host(t) for t in (bits, scales, md, ed, xd) + ((xb,) if xb is not None else ())])
        if static:
            assert int(st.item()) == 0, "a cross-workgroup wait of the allocation-free call gave up"
        else:
            assert ob.onebit_workspace_status(ws) == 0
    for name, a, b in zip(("bits", "scales", "m", "e", "x", "x_bf16"), *outs):
        assert_exact(f"static vs workspace {name}", b, a)
    return plan


def test_two_calls_second_smaller_match_the_workspace_call():
    big = ob.onebit_onepass_max_elements() + 4097
    off1 = W.offsets_from_sizes([5000, big, 3, 70001, 1 << 20])
    t1 = W.offsets_from_sizes([4000, 1000 + big, 3, 70001 + (1 << 20)])
    k1 = np.array([1, 1, 0, 1], np.uint8)
    say(f"first call: {int(off1[-1])} elements, one chunk of {big} (two-pass)")
    p1 = both(off1, t1, k1, 1)
    assert ob.onebit_plan_stats(p1)["twopass_tiles"] > 0
    off2 = W.offsets_from_sizes([33, 9000, 2048 * 7 + 5])
    say(f"second call: {int(off2[-1])} elements")
    both(off2, None, None, 2)
    both(off2, None, None, 3, update=False)
    both(np.array([0], np.int64), None, None, 4, update=False)


def test_plan_beyond_the_scratch_is_refused():
    # 2^20 chunks of 1 element: 2^20 tiles + 2^20 chunks + 1 words > 2^20
    off = np.arange(0, (1 << 20) + 1, dtype=np.int64)
    plan = ob.onebit_plan_create(off)
    with pytest.raises(ob.OnebitError) as info:
        ob.onebit_compress_update_static(plan, torch.zeros(1 << 20, device=DEV), torch.zeros(1 << 20, device=DEV),
                                         torch.zeros(1 << 20, device=DEV), None, None, None,
                                         torch.zeros(1 << 15, dtype=torch.int32, device=DEV),
                                         torch.zeros(1 << 20, device=DEV), **H)
    assert info.value.status == ob.ONEBIT_ERR_NOMEM

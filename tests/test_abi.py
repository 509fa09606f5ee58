"""Host-side checks of the C-ABI library (no kernel is launched here).

The library loads, exports every function include/onebit.h declares, and rejects
invalid arguments before touching a device.
"""
import ctypes as C

import numpy as np
import pytest

from error_compensated_bit_amd import onebit as ob


def test_library_exports_every_declared_function():
    lib = ob.load()
    names = ob.header_functions()
    assert len(names) >= 16
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(ob._SIGS), "binding and header disagree"


def test_status_strings():
    for s in range(6):
        assert ob.onebit_status_string(s)
    assert ob.onebit_status_string(99) == "unknown status"


@pytest.mark.parametrize("offsets", [[1, 5], [0, 5, 3], []])
def test_plan_rejects_bad_chunk_tables(offsets):
    lib = ob.load()
    out = C.c_void_p()
    arr = np.asarray(offsets, np.int64)
    st = lib.onebit_plan_create(arr.ctypes.data if arr.size else None, max(arr.size - 1, 0), None, None, 0,
                                C.byref(out))
    assert st == ob.ONEBIT_ERR_INVALID and not out.value


def test_plan_rejects_bad_tensor_tables():
    lib = ob.load()
    out = C.c_void_p()
    co = np.array([0, 10], np.int64)
    to = np.array([0, 4, 9], np.int64)              # does not end at n
    keep = np.array([1, 0], np.uint8)
    assert lib.onebit_plan_create(co.ctypes.data, 1, to.ctypes.data, keep.ctypes.data, 2,
                                  C.byref(out)) == ob.ONEBIT_ERR_INVALID
    assert lib.onebit_plan_create(co.ctypes.data, 1, None, keep.ctypes.data, 2, C.byref(out)) == ob.ONEBIT_ERR_INVALID
    assert lib.onebit_plan_create(co.ctypes.data, 1, None, None, 0, None) == ob.ONEBIT_ERR_INVALID


def test_calls_reject_invalid_arguments_before_any_launch():
    lib = ob.load()
    assert lib.onebit_compress_update(None, None, 0, None, None, None, None, None, None, None, 1e-3, 0.9, 1e-8, 0.0,
                                      None, None) == ob.ONEBIT_ERR_INVALID
    assert lib.onebit_server_reduce(None, 2, None, None, None, None, None, None, None, None) == ob.ONEBIT_ERR_INVALID
    assert lib.onebit_adam_warmup_step(None, None, None, None, 0, -1, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, 1,
                                       None) == ob.ONEBIT_ERR_INVALID
    assert lib.onebit_adam_warmup_step(None, None, None, None, 7, 10, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, 1,
                                       None) == ob.ONEBIT_ERR_INVALID   # bad dtype
    assert lib.qsdp_quantize(None, 10, 1024, 5, 0, None, None, None, None) == ob.ONEBIT_ERR_INVALID
    assert lib.qsdp_quantize(None, 10, 1023, 4, 0, None, None, None, None) == ob.ONEBIT_ERR_INVALID
    assert lib.qsdp_dequantize(None, None, None, 10, 0, 8, None, None, None) == ob.ONEBIT_ERR_INVALID
    # n == 0 is a no-op that succeeds without touching pointers
    assert lib.qsdp_quantize(None, 0, 1024, 4, 0, None, None, None, None) == ob.ONEBIT_OK
    assert lib.onebit_workspace_init(None, 64, None) == ob.ONEBIT_ERR_INVALID


def test_host_tensors_are_refused_before_any_launch():
    """A host tensor handed to a call would give the kernels a host address; the
    binding refuses it (no GPU needed: nothing reaches the library)."""
    import torch
    t = torch.zeros(64)
    with pytest.raises(TypeError):
        ob.onebit_momentum_update(t, None, t, t, None, lr=1e-3, eps=1e-8, weight_decay=0.0)
    with pytest.raises(TypeError):
        ob.qsdp_dequantize(torch.zeros(32, dtype=torch.uint8), t, t, 64, 32, 4, None, t)

"""Python binding of libonebit (include/onebit.h): same names, argument marshalling only.

Device buffers are torch CUDA tensors (PyTorch supplies device memory and the
stream); every computation runs in the library's HIP kernels.  A missing library
raises immediately: there is no fallback path.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os
import re
import sys
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libonebit.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "onebit.h")

ONEBIT_OK, ONEBIT_ERR_INVALID, ONEBIT_ERR_ALIGN, ONEBIT_ERR_HIP, ONEBIT_ERR_NOMEM, ONEBIT_ERR_UNSUPPORTED = range(6)
ONEBIT_F32, ONEBIT_BF16, ONEBIT_F16 = 0, 1, 2

_P, _I64, _I, _D, _U64, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_double, C.c_uint64, C.c_size_t

_SIGS = {
    "onebit_status_string": (C.c_char_p, [_I]),
    "onebit_set_spin_limit": (None, [C.c_uint32]),
    "onebit_set_grid_cap": (None, [C.c_int32]),
    "onebit_plan_create": (_I, [_P, _I64, _P, _P, _I64, C.POINTER(_P)]),
    "onebit_plan_destroy": (None, [_P]),
    "onebit_plan_host_tables": (_I, [_P, _I64, _P, _P, _I64, _P, _P, _P, _P, _P]),
    "onebit_plan_elements": (_I64, [_P]),
    "onebit_plan_chunks": (_I64, [_P]),
    "onebit_plan_words": (_I64, [_P]),
    "onebit_plan_workspace_bytes": (_SZ, [_P]),
    "onebit_workspace_init": (_I, [_P, _SZ, _P]),
    "onebit_workspace_status": (_I, [_P, C.POINTER(_U64), _P]),
    "onebit_device_resident_capacity": (C.c_int32, []),
    "onebit_plan_stats": (None, [_P, _P]),
    "onebit_onepass_max_elements": (_I64, []),
    "onebit_profile_begin": (None, []),
    "onebit_profile_begin_classes": (None, [C.c_uint32]),
    "onebit_profile_end": (_I, [_P, _P]),
    "onebit_adam_warmup_step": (_I, [_P, _P, _P, _P, _I, _I64, _D, _D, _D, _D, _D, _I, _I64, _P]),
    "onebit_compress_update": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _D, _D, _D, _D, _P, _P]),
    "onebit_compress_update_packed": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _D, _D, _D, _D, _P, _P]),
    "onebit_compress_update_static": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _D, _D, _D, _D, _P, _P]),
    "onebit_momentum_update_packed": (_I, [_P, _P, _P, _P, _P, _P, _P, _D, _D, _D, _P]),
    "onebit_server_reduce": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "onebit_stream_probe": (_I, [_P, _I, _P, _I, _I64, _I, _I, _I, _P]),
    "onebit_philox_probe": (_I, [_U64, _I64, _P, _I, _I, _P]),
    "onebit_momentum_update": (_I, [_P, _P, _P, _P, _P, _I64, _D, _D, _D, _P]),
    "onebit_decompress": (_I, [_P, _P, _P, _P, _P, _P]),
    "onebit_average_rows": (_I, [_P, _I, _I, _I64, _I64, _P, _P]),
    "qsgd_quantize": (_I, [_P, _I, _I64, _I, _I, _U64, _P, _P, _P]),
    "qsgd_reduce": (_I, [_I, _P, _I64, _P, _I64, _I64, _I, _I, _P, _P, _P]),
    "loco_quantize": (_I, [_P, _I, _P, _I64, _I, _I, _D, _U64, _P, _P, _P]),
    "qsdp_quantize": (_I, [_P, _I64, _I, _I, _U64, _P, _P, _P, _P]),
    "qsdp_dequantize": (_I, [_P, _P, _P, _I64, _I, _I, _P, _P, _P]),
    "qsdp_error_stats": (_I, [_P, _P, _I64, _P, _P, _P, _P]),
    "qsdp_mean_abs_error": (_I, [_P, _P, _I64, _I, _P, _P, _P]),
}

QSDP_STATS_PARTIALS = 1024

_lib = None


class OnebitError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {onebit_status_string(status)} (status {status})")


def load():
    """Load libonebit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback implementation")
        # torch ships its own HIP runtime; loading it first makes the library bind to
        # that same runtime (loaded the other way round, the process would hold two
        # runtimes and the library's first HIP call would fail)
        import torch  # noqa: F401
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions include/onebit.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def _check(status, what):
    if status != ONEBIT_OK:
        raise OnebitError(status, what)


def _ptr(t):
    """Device address of a tensor whose innermost dimension is dense.  Host tensors
    are refused here: the kernels would fault on a host address."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError(f"expected a device (GPU) tensor, got one on {t.device}")
    if t.numel() > 1 and t.stride(-1) != 1:
        raise ValueError("the innermost dimension of a tensor argument must be contiguous")
    if t.dim() == 1 and t.numel() > 1 and not t.is_contiguous():
        raise ValueError("one-dimensional tensor arguments must be contiguous")
    return t.data_ptr()


def _rows(t, row_len, what):
    """A [rows, row_len] tensor laid out row-major with no padding between rows."""
    if t.dim() != 2 or t.shape[1] < row_len or (t.shape[0] > 1 and t.stride(0) != row_len):
        raise ValueError(f"{what} must be a [W, {row_len}] row-major tensor with rows of exactly {row_len} entries")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return ONEBIT_F32
    if t.dtype in (torch.bfloat16, torch.int16):
        return ONEBIT_BF16
    if t.dtype == torch.float16:
        return ONEBIT_F16
    raise TypeError(f"gradient dtype {t.dtype} is not float32, bfloat16 or float16")


# ---------------------------------------------------------------- API

def onebit_status_string(status: int) -> str:
    return load().onebit_status_string(int(status)).decode()


_live_plans = weakref.WeakSet()


class Plan:
    """Owning handle of an onebit_plan_t (destroyed with the object, or at interpreter
    exit while the HIP runtime is still up; never from a finalizing interpreter)."""

    def __init__(self, handle):
        self.handle = handle
        _live_plans.add(self)

    def close(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.onebit_plan_destroy(self.handle)
        self.handle = None

    def __del__(self):
        if not sys.is_finalizing():
            self.close()


@atexit.register
def _release_plans():
    for p in list(_live_plans):
        p.close()

    @property
    def _as_parameter_(self):
        return self.handle


def onebit_plan_create(chunk_offsets, tensor_offsets=None, tensor_keep=None) -> Plan:
    lib = load()
    co = np.ascontiguousarray(chunk_offsets, dtype=np.int64)
    to = None if tensor_offsets is None else np.ascontiguousarray(tensor_offsets, dtype=np.int64)
    tk = None if tensor_keep is None else np.ascontiguousarray(tensor_keep, dtype=np.uint8)
    out = _P()
    n_tensors = 0 if to is None else to.size - 1
    _check(lib.onebit_plan_create(co.ctypes.data, co.size - 1, None if to is None else to.ctypes.data,
                                  None if tk is None else tk.ctypes.data, n_tensors, C.byref(out)),
           "onebit_plan_create")
    return Plan(out.value)


def onebit_plan_host_tables(chunk_offsets, tensor_offsets=None, tensor_keep=None):
    """Host-only plan tables: (tiles int64[n_tiles, 6], words, masked intervals int64[k, 2])."""
    lib = load()
    co = np.ascontiguousarray(chunk_offsets, dtype=np.int64)
    to = None if tensor_offsets is None else np.ascontiguousarray(tensor_offsets, dtype=np.int64)
    tk = None if tensor_keep is None else np.ascontiguousarray(tensor_keep, dtype=np.uint8)
    n_t = 0 if to is None else to.size - 1
    nt, nw, ni = C.c_int64(), C.c_int64(), C.c_int64()
    args = (co.ctypes.data, co.size - 1, None if to is None else to.ctypes.data,
            None if tk is None else tk.ctypes.data, n_t)
    _check(lib.onebit_plan_host_tables(*args, C.byref(nt), C.byref(nw), None, C.byref(ni), None),
           "onebit_plan_host_tables")
    tiles = np.zeros((nt.value, 6), dtype=np.int64)
    iv = np.zeros((ni.value, 2), dtype=np.int64)
    _check(lib.onebit_plan_host_tables(*args, None, None, tiles.ctypes.data, None, iv.ctypes.data),
           "onebit_plan_host_tables")
    return tiles, int(nw.value), iv


def onebit_plan_destroy(plan: Plan):
    load()
    plan.close()


def onebit_plan_elements(plan) -> int:
    return int(load().onebit_plan_elements(plan.handle))


def onebit_plan_chunks(plan) -> int:
    return int(load().onebit_plan_chunks(plan.handle))


def onebit_plan_words(plan) -> int:
    return int(load().onebit_plan_words(plan.handle))


def onebit_plan_workspace_bytes(plan) -> int:
    return int(load().onebit_plan_workspace_bytes(plan.handle))


def onebit_plan_stats(plan) -> dict:
    out = np.zeros(6, dtype=np.int64)
    load().onebit_plan_stats(plan.handle, out.ctypes.data)
    return dict(zip(("tiles", "onepass_tiles", "twopass_tiles", "resident_capacity", "max_chunk_tiles", "aligned"),
                    out.tolist()))


def onebit_device_resident_capacity() -> int:
    return int(load().onebit_device_resident_capacity())


def onebit_onepass_max_elements() -> int:
    return int(load().onebit_onepass_max_elements())


PROFILE_CLASSES = ("warmup", "compress_pass1", "compress_onepass", "compress_pass2", "qsdp_quantize",
                   "qsdp_dequantize", "server_pass1", "server_onepass", "server_pass2", "finalize",
                   "momentum_update", "qsgd_quantize", "qsgd_reduce", "loco_quantize")


def onebit_profile_begin(classes=None):
    """classes: names from PROFILE_CLASSES to bracket with events (None: all; an
    empty list: none)."""
    if classes is None:
        load().onebit_profile_begin()
        return
    mask = 0
    for name in classes:
        mask |= 1 << PROFILE_CLASSES.index(name)
    load().onebit_profile_begin_classes(mask)


def onebit_profile_end() -> dict:
    """{class: (total_ms, launches)} for the launches since onebit_profile_begin."""
    ms = np.zeros(len(PROFILE_CLASSES), dtype=np.float64)
    cnt = np.zeros(len(PROFILE_CLASSES), dtype=np.int64)
    _check(load().onebit_profile_end(ms.ctypes.data, cnt.ctypes.data), "onebit_profile_end")
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(PROFILE_CLASSES)}


def onebit_workspace_init(workspace, stream=None):
    _check(load().onebit_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "onebit_workspace_init")


def onebit_workspace_status(workspace, stream=None) -> int:
    out = _U64()
    _check(load().onebit_workspace_status(_ptr(workspace), C.byref(out), _stream(stream)), "onebit_workspace_status")
    return int(out.value)


def onebit_adam_warmup_step(x, m, v, g, *, lr, beta1, beta2, eps, weight_decay, bias_correction, step,
                            stream=None):
    _check(load().onebit_adam_warmup_step(_ptr(x), _ptr(m), _ptr(v), _ptr(g), _dtype_code(g), x.numel(), lr, beta1,
                                          beta2, eps, weight_decay, int(bias_correction), int(step),
                                          _stream(stream)), "onebit_adam_warmup_step")


def onebit_compress_update(plan, g, m, e, v, x, x_bf16, bits, scales, *, lr, beta1, eps, weight_decay,
                           workspace, stream=None):
    _check(load().onebit_compress_update(plan.handle, _ptr(g), _dtype_code(g), _ptr(m), _ptr(e), _ptr(v), _ptr(x),
                                         _ptr(x_bf16), _ptr(bits), _ptr(scales), lr, beta1, eps, weight_decay,
                                         _ptr(workspace), _stream(stream)), "onebit_compress_update")


def onebit_compress_update_static(plan, g, m, e, v, x, x_bf16, bits, scales, *, lr, beta1, eps, weight_decay,
                                  wait_status=None, stream=None):
    """onebit_compress_update without a workspace (the library's scratch instead);
    wait_status: optional int64 device tensor of one element."""
    _check(load().onebit_compress_update_static(plan.handle, _ptr(g), _dtype_code(g), _ptr(m), _ptr(e), _ptr(v),
                                                _ptr(x), _ptr(x_bf16), _ptr(bits), _ptr(scales), lr, beta1, eps,
                                                weight_decay, _ptr(wait_status), _stream(stream)),
           "onebit_compress_update_static")


def onebit_compress_update_packed(plan, g, m_bits, m_scales, e, v, x, x_bf16, bits, scales, *, lr, beta1, eps,
                                  weight_decay, workspace, m_mask=None, stream=None):
    _check(load().onebit_compress_update_packed(plan.handle, _ptr(g), _dtype_code(g), _ptr(m_bits), _ptr(m_scales),
                                                _ptr(m_mask), _ptr(e), _ptr(v), _ptr(x), _ptr(x_bf16), _ptr(bits),
                                                _ptr(scales), lr, beta1, eps, weight_decay, _ptr(workspace),
                                                _stream(stream)),
           "onebit_compress_update_packed")


def onebit_momentum_update_packed(plan, m_bits, m_scales, mask, v, x, x_bf16, *, lr, eps, weight_decay, stream=None):
    _check(load().onebit_momentum_update_packed(plan.handle, _ptr(m_bits), _ptr(m_scales), _ptr(mask), _ptr(v), _ptr(x),
                                                _ptr(x_bf16), lr, eps, weight_decay, _stream(stream)),
           "onebit_momentum_update_packed")


def onebit_server_reduce(plan, worker_bits, worker_scales, server_error, server_bits, server_scales, m_out,
                         workspace, stream=None):
    W = int(worker_scales.shape[0])
    _rows(worker_bits, onebit_plan_words(plan), "worker_bits")
    _rows(worker_scales, onebit_plan_chunks(plan), "worker_scales")
    _check(load().onebit_server_reduce(plan.handle, W, _ptr(worker_bits), _ptr(worker_scales), _ptr(server_error),
                                       _ptr(server_bits), _ptr(server_scales), _ptr(m_out), _ptr(workspace),
                                       _stream(stream)), "onebit_server_reduce")


def onebit_stream_probe(inputs, outputs, grid, block=256, policy=1, stream=None):
    """inputs / outputs: lists of equally long fp32 device tensors (one of the mixes
    the library supports); block: threads per workgroup (256, 512 or 1024); policy:
    0 default cache policy, 1 (or True) nontemporal, 2 nontemporal loads staged in
    LDS by the load unit (256-thread workgroups, at least one input)."""
    import torch
    dev = (inputs or outputs)[0].device
    n = (inputs or outputs)[0].numel()
    pin = torch.tensor([t.data_ptr() for t in inputs] or [0], dtype=torch.int64, device=dev)
    pout = torch.tensor([t.data_ptr() for t in outputs] or [0], dtype=torch.int64, device=dev)
    _check(load().onebit_stream_probe(_ptr(pin), len(inputs), _ptr(pout), len(outputs), n, int(grid),
                                      int(block), int(policy), _stream(stream)), "onebit_stream_probe")
    return pin, pout           # keep the pointer arrays alive until the launch has run


def onebit_philox_probe(seed, n_blocks, out, grid, block=256, stream=None):
    """out: int32/uint32 device tensor of grid * block words (one XOR-folded word per thread)."""
    if out.numel() != grid * block:
        raise ValueError("out must hold grid * block words")
    _check(load().onebit_philox_probe(int(seed), int(n_blocks), _ptr(out), int(grid), int(block), _stream(stream)),
           "onebit_philox_probe")


def onebit_set_spin_limit(limit: int) -> None:
    load().onebit_set_spin_limit(int(limit))


def onebit_set_grid_cap(cap: int) -> None:
    load().onebit_set_grid_cap(int(cap))


def onebit_momentum_update(m, mask, v, x, x_bf16, *, lr, eps, weight_decay, stream=None):
    """mask: uint8 (or bool) tensor of n elements, or None."""
    _check(load().onebit_momentum_update(_ptr(m), _ptr(mask), _ptr(v), _ptr(x), _ptr(x_bf16), x.numel(), lr, eps,
                                         weight_decay, _stream(stream)), "onebit_momentum_update")


def onebit_decompress(plan, bits, scales, mask, out, stream=None):
    _check(load().onebit_decompress(plan.handle, _ptr(bits), _ptr(scales), _ptr(mask), _ptr(out), _stream(stream)),
           "onebit_decompress")


def onebit_average_rows(g, out, stream=None):
    """g: [W, n] (or 1-D for one row) fp32, bf16 or fp16 tensor with contiguous rows; out: fp32 [n]."""
    W = g.shape[0] if g.dim() == 2 else 1
    n = g.shape[-1]
    stride = g.stride(0) if g.dim() == 2 else n
    _check(load().onebit_average_rows(_ptr(g), _dtype_code(g), W, stride, n, _ptr(out), _stream(stream)),
           "onebit_average_rows")


def qsgd_quantize(g, bucket, bits, seed, codes, norms, stream=None):
    _check(load().qsgd_quantize(_ptr(g), _dtype_code(g), g.numel(), int(bucket), int(bits), int(seed) & (2 ** 64 - 1),
                                _ptr(codes), _ptr(norms), _stream(stream)), "qsgd_quantize")


def loco_quantize(g, err_avg, bucket, bits, beta, seed, codes, norms, stream=None):
    _check(load().loco_quantize(_ptr(g), _dtype_code(g), _ptr(err_avg), g.numel(), int(bucket), int(bits), float(beta),
                                int(seed) & (2 ** 64 - 1), _ptr(codes), _ptr(norms), _stream(stream)), "loco_quantize")


def qsgd_reduce(codes, norms, n, bucket, bits, out_f32=None, out_bf16=None, stream=None):
    """codes: uint8 [W, stride] (or 1-D for one worker); norms: float32 [W, stride] (or 1-D)."""
    W = codes.shape[0] if codes.dim() == 2 else 1
    cs = codes.stride(0) if codes.dim() == 2 else 0
    ns = norms.stride(0) if norms.dim() == 2 else 0
    _check(load().qsgd_reduce(W, _ptr(codes), cs, _ptr(norms), ns, int(n), int(bucket), int(bits), _ptr(out_f32),
                              _ptr(out_bf16), _stream(stream)), "qsgd_reduce")


def qsdp_quantize(x_bf16, bucket, bits, seed, codes, bucket_min, bucket_max, stream=None):
    _check(load().qsdp_quantize(_ptr(x_bf16), x_bf16.numel(), int(bucket), int(bits), int(seed) & (2 ** 64 - 1),
                                _ptr(codes), _ptr(bucket_min), _ptr(bucket_max), _stream(stream)), "qsdp_quantize")


def qsdp_dequantize(codes, bucket_min, bucket_max, n, bucket, bits, out_bf16=None, out_f32=None, stream=None):
    _check(load().qsdp_dequantize(_ptr(codes), _ptr(bucket_min), _ptr(bucket_max), int(n), int(bucket), int(bits),
                                  _ptr(out_bf16), _ptr(out_f32), _stream(stream)), "qsdp_dequantize")


def qsdp_error_stats(x_bf16, y, ysum, sums, partials, stream=None):
    _check(load().qsdp_error_stats(_ptr(x_bf16), _ptr(y), y.numel(), _ptr(ysum), _ptr(sums), _ptr(partials),
                                   _stream(stream)), "qsdp_error_stats")


def qsdp_mean_abs_error(x_bf16, ysum, seeds, out, partials, stream=None):
    _check(load().qsdp_mean_abs_error(_ptr(x_bf16), _ptr(ysum), ysum.numel(), int(seeds), _ptr(out), _ptr(partials),
                                      _stream(stream)), "qsdp_mean_abs_error")

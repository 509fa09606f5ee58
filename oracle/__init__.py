"""Python view of the CPU oracle (oracle/onebit_oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the product library never does.

Every function takes and returns numpy arrays, copies nothing it does not have
to, and raises on a non-zero status.  The arithmetic lives in C; this module
only marshals arguments (and widens bf16 gradients, which is exact).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB selects another build of the same source (the sanitizer tests run the
# pins against an -fsanitize=undefined build this way)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_P = C.c_void_p
_I64 = C.c_int64
_F = C.c_float
_D = C.c_double
_I = C.c_int


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = C.CDLL(_LIB_PATH)
        lib.oracle_adam_warmup_step.argtypes = [_P, _P, _P, _P, _I64, _D, _D, _D, _D, _D, _I, _I64]
        lib.oracle_compress_update.argtypes = [_P, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _D, _D, _D, _D, _I]
        lib.oracle_server_reduce.argtypes = [_P, _I64, _I, _P, _P, _P, _P, _P, _P]
        lib.oracle_decompress.argtypes = [_P, _I64, _P, _P, _P]
        lib.oracle_qsgd_quantize.argtypes = [_P, _I, _I64, _I, _I, C.c_uint64, _I64, _P, _P]
        lib.oracle_qsgd_reduce.argtypes = [_I, _P, _I64, _P, _I64, _I64, _I, _I, _P, _P]
        lib.oracle_loco_quantize.argtypes = [_P, _I, _P, _I64, _I, _I, _D, C.c_uint64, _I64, _P, _P]
        lib.oracle_momentum_update.argtypes = [_P, _P, _P, _P, _P, _I64, _D, _D, _D]
        lib.oracle_average_rows.argtypes = [_P, _I, _I64, _I64, _P]
        lib.oracle_philox4x32_10.argtypes = [_P, _P, _P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_qsdp_uniform.argtypes = [C.c_uint64, _I64]
        lib.oracle_qsdp_uniform.restype = C.c_uint32
        lib.oracle_qsdp_quantize.argtypes = [_P, _I64, _I, _I, C.c_uint64, _I64, _P, _P, _P]
        lib.oracle_qsdp_dequantize.argtypes = [_P, _P, _P, _I64, _I, _I, _P, _P]
        lib.oracle_f32_to_bf16.argtypes = [_F]
        lib.oracle_f32_to_bf16.restype = C.c_uint16
        for name in ("oracle_adam_warmup_step", "oracle_compress_update", "oracle_server_reduce",
                     "oracle_momentum_update", "oracle_qsgd_quantize", "oracle_qsgd_reduce",
                     "oracle_loco_quantize", "oracle_average_rows",
                     "oracle_decompress", "oracle_qsdp_quantize", "oracle_qsdp_dequantize"):
            getattr(lib, name).restype = C.c_int
        _lib = lib
    return _lib


class use_library:
    """Context manager: route every call through another build of the oracle source.

    Used by the mutation tests, which compile deliberately broken copies of the
    oracle and check that the pins reject them.
    """

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib, _LIB_PATH
        self._saved = (_lib, _LIB_PATH)
        _lib, _LIB_PATH = None, self.path
        _load()
        return self

    def __exit__(self, *exc):
        global _lib, _LIB_PATH
        _lib, _LIB_PATH = self._saved
        return False


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def _check(status, what):
    if status != 0:
        raise RuntimeError(f"oracle {what} failed with status {status}")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _widen(g):
    """Exact widening of a gradient given as float32, bfloat16 bits (uint16) or float16."""
    if g.dtype == np.uint16:
        return bf16_bits_to_f32(g)
    if g.dtype == np.float16:
        return np.ascontiguousarray(g, dtype=np.float32)
    return _f32(g)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns, via the C oracle helper."""
    lib = _load()
    x = _f32(x).ravel()
    return np.fromiter((lib.oracle_f32_to_bf16(float(v)) for v in x), dtype=np.uint16, count=x.size)


def words_for_chunks(chunk_off: np.ndarray) -> int:
    lens = np.diff(np.asarray(chunk_off, dtype=np.int64))
    return int(((lens + 31) // 32).sum())


def adam_warmup_step(x, m, v, g, *, lr, beta1, beta2, eps, weight_decay, bias_correction, step):
    """In place on float32 arrays x, m, v; g is float32 (or uint16 bf16 bits)."""
    lib = _load()
    g = _widen(g)
    _check(lib.oracle_adam_warmup_step(_ptr(x), _ptr(m), _ptr(v), _ptr(g), x.size, lr, beta1, beta2,
                                       eps, weight_decay, int(bias_correction), int(step)), "warmup")


def compress_update(chunk_off, g, m, e, v=None, x=None, *, tensor_off=None, tensor_keep=None,
                    lr=0.0, beta1=0.9, eps=1e-8, weight_decay=0.0, want_bf16=False, identity=False):
    """Worker compression (+ frozen-v update when v and x are given), in place on m, e, x.

    Returns (bits uint32[plan_words], scales float32[n_chunks], x_bf16 uint16[n] or None).
    """
    lib = _load()
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int64)
    n_chunks = chunk_off.size - 1
    g = _widen(g)
    bits = np.zeros(max(words_for_chunks(chunk_off), 1), dtype=np.uint32)
    scales = np.zeros(max(n_chunks, 1), dtype=np.float32)
    xb = np.zeros(x.size, dtype=np.uint16) if (want_bf16 and x is not None) else None
    if tensor_off is not None:
        tensor_off = np.ascontiguousarray(tensor_off, dtype=np.int64)
        tensor_keep = np.ascontiguousarray(tensor_keep, dtype=np.uint8)
        n_tensors = tensor_off.size - 1
    else:
        n_tensors = 0
    _check(lib.oracle_compress_update(_ptr(chunk_off), n_chunks, _ptr(tensor_off), _ptr(tensor_keep), n_tensors,
                                      _ptr(g), _ptr(m), _ptr(e), _ptr(v), _ptr(x), _ptr(xb), _ptr(bits),
                                      _ptr(scales), lr, beta1, eps, weight_decay, int(identity)), "compress")
    return bits[:words_for_chunks(chunk_off)], scales[:n_chunks], xb


def server_reduce(chunk_off, worker_bits, worker_scales, server_error, *, want_m=True):
    """Server stage over W workers.  worker_bits uint32[W, plan_words], worker_scales float32[W, n_chunks].

    server_error is updated in place.  Returns (bits, scales, m_out or None).
    """
    lib = _load()
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int64)
    n_chunks = chunk_off.size - 1
    worker_bits = np.ascontiguousarray(worker_bits, dtype=np.uint32)
    worker_scales = np.ascontiguousarray(worker_scales, dtype=np.float32)
    W = worker_bits.shape[0]
    bits = np.zeros(max(words_for_chunks(chunk_off), 1), dtype=np.uint32)
    scales = np.zeros(max(n_chunks, 1), dtype=np.float32)
    m_out = np.zeros(server_error.size, dtype=np.float32) if want_m else None
    _check(lib.oracle_server_reduce(_ptr(chunk_off), n_chunks, W, _ptr(worker_bits), _ptr(worker_scales),
                                    _ptr(server_error), _ptr(bits), _ptr(scales), _ptr(m_out)), "server")
    return bits[:words_for_chunks(chunk_off)], scales[:n_chunks], m_out


def momentum_update(m, v, x, *, mask=None, lr, eps, weight_decay, want_bf16=False):
    """Worker finish after the all-reduce, in place on m and x.  Returns x_bf16 or None."""
    lib = _load()
    mask = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    xb = np.zeros(x.size, dtype=np.uint16) if want_bf16 else None
    _check(lib.oracle_momentum_update(_ptr(m), _ptr(mask), _ptr(v), _ptr(x), _ptr(xb), x.size, lr, eps,
                                      weight_decay), "momentum_update")
    return xb


def decompress(chunk_off, bits, scales):
    lib = _load()
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int64)
    out = np.zeros(int(chunk_off[-1]), dtype=np.float32)
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    _check(lib.oracle_decompress(_ptr(chunk_off), chunk_off.size - 1, _ptr(bits), _ptr(scales), _ptr(out)),
           "decompress")
    return out


def philox4x32_10(key, ctr):
    lib = _load()
    k = np.ascontiguousarray(key, dtype=np.uint32)
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(k), _ptr(c), _ptr(out))
    return out


def qsdp_uniform(seed: int, i: int) -> int:
    return int(_load().oracle_qsdp_uniform(seed, i))


def qsdp_quantize(x_bf16, *, bucket, bits, seed, first_index=0):
    """x_bf16: uint16 bit patterns (global indices first_index...).  Returns (codes, bucket_min, bucket_max)."""
    lib = _load()
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n = x_bf16.size
    nb = (n + bucket - 1) // bucket
    codes = np.zeros(max((n + 1) // 2 if bits == 4 else n, 1), dtype=np.uint8)
    bmin = np.zeros(max(nb, 1), dtype=np.float32)
    bmax = np.zeros(max(nb, 1), dtype=np.float32)
    _check(lib.oracle_qsdp_quantize(_ptr(x_bf16), n, bucket, bits, seed, first_index, _ptr(codes), _ptr(bmin),
                                    _ptr(bmax)),
           "qsdp_quantize")
    return codes[:((n + 1) // 2 if bits == 4 else n)], bmin[:nb], bmax[:nb]


def qsdp_dequantize(codes, bmin, bmax, n, *, bucket, bits, want_f32=False):
    """Returns (y_bf16 uint16[n], y_f32 float32[n] or None)."""
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    bmin = _f32(bmin)
    bmax = _f32(bmax)
    out = np.zeros(max(n, 1), dtype=np.uint16)
    y = np.zeros(max(n, 1), dtype=np.float32) if want_f32 else None
    _check(lib.oracle_qsdp_dequantize(_ptr(codes), _ptr(bmin), _ptr(bmax), n, bucket, bits, _ptr(out), _ptr(y)),
           "qsdp_dequantize")
    return out[:n], (y[:n] if want_f32 else None)


def qsgd_quantize(g, *, bucket, bits, seed, first_index=0):
    """g: float32 values or bf16 bit patterns (uint16), global indices first_index...
    Returns (codes, norms)."""
    lib = _load()
    if g.dtype == np.uint16:
        dt = 1
    else:
        g = _widen(g)
        dt = 0
    g = np.ascontiguousarray(g)
    n = g.size
    nb = (n + bucket - 1) // bucket
    nbytes = (n + 1) // 2 if bits == 4 else n
    codes = np.zeros(max(nbytes, 1), dtype=np.uint8)
    norms = np.zeros(max(nb, 1), dtype=np.float32)
    _check(lib.oracle_qsgd_quantize(_ptr(g), dt, n, bucket, bits, seed, first_index, _ptr(codes), _ptr(norms)),
           "qsgd_quantize")
    return codes[:nbytes], norms[:nb]


def qsgd_reduce(codes, norms, n, *, bucket, bits, want_bf16=False):
    """codes: uint8 [W, code_bytes] (or 1-D for one worker); norms: float32 [W, n_buckets].
    Returns (y_f32 [n], y_bf16 [n] or None)."""
    lib = _load()
    codes = np.ascontiguousarray(np.atleast_2d(codes), dtype=np.uint8)
    norms = np.ascontiguousarray(np.atleast_2d(norms), dtype=np.float32)
    W = codes.shape[0]
    out = np.zeros(max(n, 1), dtype=np.float32)
    ob = np.zeros(max(n, 1), dtype=np.uint16) if want_bf16 else None
    _check(lib.oracle_qsgd_reduce(W, _ptr(codes), codes.shape[1], _ptr(norms), norms.shape[1], n, bucket, bits,
                                  _ptr(out), _ptr(ob)), "qsgd_reduce")
    return out[:n], (ob[:n] if want_bf16 else None)


def loco_quantize(g, err_avg, *, bucket, bits, beta, seed, first_index=0):
    """LoCo-style step, err_avg (float32) updated in place.  Returns (codes, norms)."""
    lib = _load()
    if g.dtype == np.uint16:
        dt = 1
    else:
        g = _widen(g)
        dt = 0
    g = np.ascontiguousarray(g)
    n = g.size
    nb = (n + bucket - 1) // bucket
    nbytes = (n + 1) // 2 if bits == 4 else n
    codes = np.zeros(max(nbytes, 1), dtype=np.uint8)
    norms = np.zeros(max(nb, 1), dtype=np.float32)
    _check(lib.oracle_loco_quantize(_ptr(g), dt, _ptr(err_avg), n, bucket, bits, beta, seed, first_index,
                                    _ptr(codes), _ptr(norms)), "loco_quantize")
    return codes[:nbytes], norms[:nb]


def average_rows(g):
    """Mean over the rows of g ([W, n] float32, or bf16 bit patterns as uint16, widened
    exactly) as the warmup phase's full-precision exchange forms it.  Returns fp32 [n]."""
    lib = _load()
    g = np.atleast_2d(g)
    if g.dtype == np.uint16:
        g = (g.astype(np.uint32) << 16).view(np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    W, n = g.shape
    out = np.zeros(max(n, 1), dtype=np.float32)
    _check(lib.oracle_average_rows(_ptr(g), W, n, n, _ptr(out)), "average_rows")
    return out[:n]

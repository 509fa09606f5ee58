"""Comparison rules shared by the GPU parity tests (HIP library vs CPU oracle).

  bits, codes, bucket min/max          exact
  scales                               exact expected; |d| <= 1e-5 |ref| tolerated and counted
  m (and warmup m, v)                  |d| <= 1e-5 |ref|; masked m exactly 0
  e, server error                      |d| <= 1e-5 max(|ref|, scale of the chunk); masked e exactly 0
  x                                    |d| <= 1e-5 max(|x_ref|, |x_ref - x_prev|)
  bf16 outputs                         <= 1 bf16 ulp
"""
import sys

import numpy as np
import torch


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def assert_exact(name, got, ref):
    """Bit-pattern equality (so -0 != +0 and NaN payloads count)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert got.dtype.itemsize == ref.dtype.itemsize, (name, got.dtype, ref.dtype)
    bad = np.nonzero(_bits(got) != _bits(ref))[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{name}: {bad.size} mismatches, first at {i.tolist()}: got {got[i]} want {ref[i]}")


def assert_bits_exact(name, got, ref):
    assert_exact(name, np.asarray(got).view(np.uint32), np.asarray(ref).view(np.uint32))


def check_scales(name, got, ref):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 * np.abs(ref.astype(np.float64))), name
    return int((got != ref).sum())


def check_rel(name, got, ref, rtol=1e-5):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    bad = np.nonzero(d > rtol * np.abs(ref))[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{name}: {bad.size} beyond rel {rtol}, first {i.tolist()}: got {got[i]} want {ref[i]}")


def check_err(name, got, ref, scale_per_el):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = 1e-5 * np.maximum(np.abs(ref), np.abs(scale_per_el))
    bad = np.nonzero(np.abs(got - ref) > tol)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{name}: {bad.size} beyond tolerance, first {i.tolist()}: got {got[i]} want {ref[i]}")


def check_x(name, got, ref, prev):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    prev = np.asarray(prev, np.float64)
    tol = 1e-5 * np.maximum(np.abs(ref), np.abs(ref - prev))
    bad = np.nonzero(np.abs(got - ref) > tol)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{name}: {bad.size} beyond tolerance, first {i.tolist()}: got {got[i]} want {ref[i]}")


def _bf16_key(p):
    p = np.asarray(p).astype(np.int64)
    return np.where(p & 0x8000, -(p & 0x7FFF), p)   # monotone in the value; +0 and -0 both 0


def check_bf16(name, got_u16, ref_u16):
    g = _bf16_key(got_u16)
    r = _bf16_key(ref_u16)
    bad = np.nonzero(np.abs(g - r) > 1)[0]
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{name}: {bad.size} beyond 1 bf16 ulp, first {i.tolist()}: {g[i]} vs {r[i]}")


def per_element(values, chunk_off):
    return np.repeat(np.asarray(values, np.float64), np.diff(np.asarray(chunk_off)))


def local_tensor_table(tensor_off, tensor_keep, lo, hi):
    """Tensors intersecting [lo, hi), clipped and shifted to start at 0."""
    if tensor_off is None:
        return None, None
    to = np.asarray(tensor_off)
    first = int(np.searchsorted(to, lo, side="right") - 1)
    last = int(np.searchsorted(to, hi, side="left"))
    bounds = np.clip(to[first:last + 1], lo, hi) - lo
    keep = np.asarray(tensor_keep)[first:last]
    return bounds.astype(np.int64), keep.astype(np.uint8)

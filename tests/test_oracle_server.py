"""Pins for the oracle's server stage of the compressed all-reduce.

Source: DeepSpeed 1-bit Adam guide sec. 4 (worker_error and server_error; the
server averages the workers' compressed momenta and compresses the average again
with its own error buffer); 1-bit Adam review, "proposed method".

Pinned by brute force on tiny inputs (numpy unpacks every worker's bits, averages
in fp64, compresses with packbits / math.fsum) and by the W = 1 special case, in
which the server recompresses a single decompressed worker stream and must
reproduce that worker's bits and scale with zero error.
"""
import math

import numpy as np
import pytest

import oracle
from error_compensated_bit_amd import workloads as W

LENGTHS = [33, 64, 1, 1000, 4097, 31]


def unpack(bits, chunk_off):
    out = []
    wbase = 0
    for j in range(chunk_off.size - 1):
        ln = int(chunk_off[j + 1] - chunk_off[j])
        nw = (ln + 31) // 32
        b = np.unpackbits(bits[wbase:wbase + nw].view(np.uint8), bitorder="little")[:ln]
        out.append(b.astype(bool))
        wbase += nw
    return np.concatenate(out)


def worker_streams(off, W_, rng):
    n = int(off[-1])
    bits, scales = [], []
    for w in range(W_):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32)
        m = np.zeros(n, np.float32)
        e = np.zeros(n, np.float32)
        b, s, _ = oracle.compress_update(off, g, m, e, beta1=0.0)     # compress-only, c = g
        bits.append(b)
        scales.append(s)
    return np.stack(bits), np.stack(scales)


@pytest.mark.parametrize("W_", [1, 2, 3, 16])
def test_server_brute_force(W_):
    rng = np.random.default_rng(10 + W_)
    off = W.offsets_from_sizes(LENGTHS)
    n = int(off[-1])
    wb, ws = worker_streams(off, W_, rng)
    es = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    es_ref = es.copy()
    bits, scales, m_out = oracle.server_reduce(off, wb, ws, es)

    # brute force: decompress every worker to fp64, average, add e_s in fp32
    dec = np.zeros((W_, n))
    for w in range(W_):
        neg = unpack(wb[w], off)
        per_el = np.repeat(ws[w].astype(np.float64), np.diff(off))
        dec[w] = np.where(neg, -per_el, per_el)
    a = np.zeros(n)
    for w in range(W_):                      # fp64 sum in worker order
        a = a + dec[w]
    c = (a / W_).astype(np.float32) + es_ref   # one rounding, then an fp32 add
    for j in range(len(LENGTHS)):
        lo, hi = off[j], off[j + 1]
        s = math.fsum(float(v) ** 2 for v in c[lo:hi].astype(np.float64))
        assert scales[j] == np.float32(math.sqrt(s) / math.sqrt(hi - lo))
    neg = c < 0
    np.testing.assert_array_equal(unpack(bits, off), neg)
    q = np.where(neg, -np.repeat(scales, np.diff(off)), np.repeat(scales, np.diff(off))).astype(np.float32)
    np.testing.assert_array_equal(m_out, q)
    np.testing.assert_array_equal(es, c - q)


def test_single_worker_server_reproduces_worker_stream():
    rng = np.random.default_rng(99)
    off = W.offsets_from_sizes(LENGTHS)
    n = int(off[-1])
    wb, ws = worker_streams(off, 1, rng)
    es = np.zeros(n, np.float32)
    bits, scales, m_out = oracle.server_reduce(off, wb, ws, es)
    np.testing.assert_array_equal(bits, wb[0])
    np.testing.assert_array_equal(scales, ws[0])
    assert np.all(es == 0)
    np.testing.assert_array_equal(m_out, oracle.decompress(off, wb[0], ws[0]))


def test_decompress_matches_unpackbits():
    rng = np.random.default_rng(7)
    off = W.offsets_from_sizes(LENGTHS)
    n = int(off[-1])
    words = int(((np.diff(off) + 31) // 32).sum())
    bits = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    scales = rng.uniform(0, 1, size=len(LENGTHS)).astype(np.float32)
    y = oracle.decompress(off, bits, scales)
    per = np.repeat(scales, np.diff(off))
    np.testing.assert_array_equal(y, np.where(unpack(bits, off), -per, per))


def test_worker_server_finish_composition_equals_fused_step():
    """One worker, zero server error, no mask: compress-only -> server -> finish
    reproduces the fused compress+update bit for bit (bits, scales, m, e, x)."""
    rng = np.random.default_rng(123)
    off = W.offsets_from_sizes(LENGTHS)
    n = int(off[-1])
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    e = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = (rng.uniform(0.5, 2, n) * 1e-6).astype(np.float32)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    h = dict(lr=1e-3, eps=1e-8, weight_decay=0.01)
    fm, fe, fx = m.copy(), e.copy(), x.copy()
    fb, fs, fxb = oracle.compress_update(off, g, fm, fe, v, fx, beta1=0.9, want_bf16=True, **h)
    wm, we, wx = m.copy(), e.copy(), x.copy()
    wb, wsc, _ = oracle.compress_update(off, g, wm, we, beta1=0.9)
    es = np.zeros(n, np.float32)
    sb, ss, m_out = oracle.server_reduce(off, wb[None], wsc[None], es)
    xb = oracle.momentum_update(m_out, v, wx, want_bf16=True, **h)
    for a, b in ((wb, fb), (sb, fb), (wsc, fs), (ss, fs), (we, fe), (m_out, fm), (wx, fx), (xb, fxb)):
        np.testing.assert_array_equal(a, b)
    assert np.all(es == 0)


def test_momentum_update_mask_and_closed_form():
    """Mask zeros give m = 0 (sign of the product kept) and, with wd = 0, an unchanged x;
    with weight decay only (m = 0 everywhere) x follows x (1 - lr wd) to one rounding."""
    rng = np.random.default_rng(5)
    n = 5000
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.uniform(0.5, 2, n) * 1e-6).astype(np.float32)
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    mask = (rng.random(n) < 0.7).astype(np.uint8)
    m2, x2 = m.copy(), x.copy()
    oracle.momentum_update(m2, v, x2, mask=mask, lr=1e-3, eps=1e-8, weight_decay=0.0)
    assert np.all(m2[mask == 0] == 0) and np.array_equal(np.signbit(m2[mask == 0]), np.signbit(m[mask == 0]))
    np.testing.assert_array_equal(m2[mask == 1], m[mask == 1])
    np.testing.assert_array_equal(x2[mask == 0], x[mask == 0])
    z, x3 = np.zeros(n, np.float32), x.copy()
    oracle.momentum_update(z, v, x3, lr=1e-3, eps=1e-8, weight_decay=0.01)
    ref = x.astype(np.float64) * (1 - float(np.float32(1e-3)) * float(np.float32(0.01)))
    assert np.all(np.abs(x3 - ref) <= 2 ** -22 * np.abs(ref))

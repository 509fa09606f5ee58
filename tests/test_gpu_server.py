"""GPU parity of the simulated compressed all-reduce: W workers' compress-only
steps (each with its own error buffer, a shared momentum) followed by the server
stage, against the oracle, over 3 steps in which the server's decompressed
result becomes the shared momentum."""
import numpy as np
import pytest
import torch

from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, CompressBuffers, host, oracle_compress
import oracle
from parity import assert_bits_exact, assert_exact, check_err, check_scales, per_element, say

pytestmark = pytest.mark.gpu


def run_allreduce(chunk_off, Wn, steps, seed):
    buf = CompressBuffers(chunk_off)
    n, words, nch = buf.n, buf.words, buf.n_chunks
    rng = np.random.default_rng(seed)
    m = np.zeros(n, np.float32)
    e = [(rng.standard_normal(n) * 1e-5).astype(np.float32) for _ in range(Wn)]
    es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    md = torch.from_numpy(m.copy()).to(DEV)
    ed = [torch.from_numpy(a.copy()).to(DEV) for a in e]
    esd = torch.from_numpy(es.copy()).to(DEV)
    wbits = torch.zeros((Wn, max(words, 1)), dtype=torch.int32, device=DEV)
    wscales = torch.zeros((Wn, max(nch, 1)), dtype=torch.float32, device=DEV)
    sbits = torch.zeros(max(words, 1), dtype=torch.int32, device=DEV)
    sscales = torch.zeros(max(nch, 1), dtype=torch.float32, device=DEV)
    for s in range(steps):
        say(f"  W={Wn} step {s}")
        ref_b, ref_s = [], []
        for w in range(Wn):
            g = (np.random.default_rng(seed * 1000 + 100 * w + s).standard_normal(n) * 1e-3).astype(np.float32)
            buf.bits = wbits[w]
            buf.scales = wscales[w]
            buf.step(torch.from_numpy(g).to(DEV), md, ed[w])
            rb, rs, _ = oracle_compress(chunk_off, g, m, e[w])
            ref_b.append(rb)
            ref_s.append(rs)
        torch.cuda.synchronize()
        for w in range(Wn):
            assert_bits_exact(f"worker {w} bits", host(wbits[w])[:words].view(np.uint32), ref_b[w])
            assert check_scales(f"worker {w} scales", host(wscales[w])[:nch], ref_s[w]) == 0
            assert_exact(f"worker {w} e", host(ed[w]), e[w])
        ob.onebit_server_reduce(buf.plan, wbits, wscales, esd, sbits, sscales, md, buf.ws)
        rb, rs, m_out = oracle.server_reduce(chunk_off, np.stack(ref_b), np.stack(ref_s), es)
        torch.cuda.synchronize()
        assert_bits_exact("server bits", host(sbits)[:words].view(np.uint32), rb)
        ne = check_scales("server scales", host(sscales)[:nch], rs)
        check_err("server e", host(esd), es, per_element(rs, chunk_off))
        if ne == 0:
            assert_exact("server e", host(esd), es)
            assert_exact("server m", host(md), m_out)
        m = m_out
        assert ob.onebit_workspace_status(buf.ws) == 0


@pytest.mark.parametrize("Wn", [1, 2, 3, 16])
def test_server_ragged_chunks(Wn):
    off = W.offsets_from_sizes([33, 64, 1, 4097, 70000, 31, 8192])
    run_allreduce(off, Wn, 3, seed=40 + Wn)


def test_server_two_pass_chunk():
    off = W.offsets_from_sizes([max(ob.onebit_onepass_max_elements(), 1) + 4097, 5000])
    run_allreduce(off, 2, 2, seed=77)


def _scale_cases(rng, Wn):
    """Worker scales per chunk: a common exponent field (the exact integer sum applies),
    mixed exponents, zeros, subnormals next to the smallest normals, a negative and a
    negative-zero scale, very large scales."""
    f32 = np.float32
    cases = [
        (2.0 ** -10 * rng.uniform(1, 2, Wn)).astype(f32),                      # one exponent
        (2.0 ** -10 * rng.uniform(0.5, 2, Wn)).astype(f32),                    # mixed
        np.where(rng.random(Wn) < 0.3, 0.0, 2.0 ** -7 * rng.uniform(1, 2, Wn)).astype(f32),
        np.zeros(Wn, f32),
        (rng.integers(1, 1 << 24, Wn) * 2.0 ** -149).astype(f32),              # subnormal and smallest normal binade
        (2.0 ** 100 * rng.uniform(1, 2, Wn)).astype(f32),
        (2.0 ** -3 * rng.uniform(1, 2, Wn)).astype(f32),
        (2.0 ** -3 * rng.uniform(1, 2, Wn)).astype(f32),
    ]
    cases[6][Wn // 2] = -cases[6][Wn // 2]
    cases[7][0] = -0.0
    return cases


@pytest.mark.parametrize("Wn", [1, 3, 16, 17])
def test_server_scale_exponent_cases(Wn):
    sizes = [4096, 2048 * 3 + 5, 31, 4096 + 64, 8192, 2053, 4096, 999]
    off = W.offsets_from_sizes(sizes)
    buf = CompressBuffers(off)
    n, words, nch = buf.n, buf.words, buf.n_chunks
    rng = np.random.default_rng(900 + Wn)
    wb = rng.integers(0, 1 << 32, size=(Wn, words), dtype=np.uint64).astype(np.uint32)
    sc = np.stack(_scale_cases(rng, Wn), axis=1)  # [Wn, nch]
    assert sc.shape == (Wn, nch)
    es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    say(f"server scale cases W={Wn}")
    wbd = torch.from_numpy(wb.view(np.int32).copy()).to(DEV)
    scd = torch.from_numpy(sc.copy()).to(DEV)
    esd = torch.from_numpy(es.copy()).to(DEV)
    sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sscales = torch.zeros(nch, dtype=torch.float32, device=DEV)
    md = torch.zeros(n, dtype=torch.float32, device=DEV)
    for step in range(2):
        ob.onebit_server_reduce(buf.plan, wbd, scd, esd, sbits, sscales, md, buf.ws)
        rb, rs, m_out = oracle.server_reduce(off, wb, sc, es)
        torch.cuda.synchronize()
        assert_bits_exact(f"server bits step {step}", host(sbits).view(np.uint32), rb)
        assert check_scales(f"server scales step {step}", host(sscales), rs) == 0
        assert_exact(f"server e step {step}", host(esd), es)
        assert_exact(f"server m step {step}", host(md), m_out)
        assert ob.onebit_workspace_status(buf.ws) == 0


def _boundary_cases(rng, Wn):
    """Worker scales per chunk around the server's exact-sum condition (every scale
    finite and an exponent-field spread of at most 29 - ceil(log2 W)): the widest
    spread that still qualifies, with full mantissas at the top and an odd one at the
    bottom so that the sums need all 53 bits; one step wider; a spread of 40, where
    the ordered sum does round; the subnormal floor at the widest qualifying spread;
    an infinite and a NaN scale; signed zeros; equal scales."""
    f32 = np.float32
    lg = int(np.ceil(np.log2(Wn))) if Wn > 1 else 0
    d = 29 - lg

    def spread(top_exp, width):
        s = np.ldexp(rng.uniform(1, 2, Wn), rng.integers(top_exp - width, top_exp + 1, Wn)).astype(f32)
        s[0] = np.float32(np.ldexp(2.0 - 2.0 ** -23, top_exp))
        if Wn > 1:
            s[-1] = np.float32(np.ldexp(1.0 + 2.0 ** -23, top_exp - width))
        return s

    cases = [spread(0, d), spread(-3, d + 1), spread(5, 40)]
    floor = spread(-126 + d, d)                                  # lowest field 1 (smallest normals)
    if Wn > 1:
        floor[-1] = np.float32(2.0 ** -149)                      # a subnormal counts as field 1
    cases.append(floor)
    inf_case = spread(-2, 3)
    inf_case[Wn // 2] = np.inf
    nan_case = spread(-2, 3)
    nan_case[0] = np.nan
    zeros = spread(-8, 2)
    zeros[0] = -0.0
    if Wn > 2:
        zeros[1] = 0.0
    cases += [inf_case, nan_case, zeros, np.full(Wn, 2.0 ** -9 * 1.375, f32)]
    return cases


def _assert_same_or_both_nan(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), (name, int(np.isnan(got).sum()), int(nan.sum()))
    assert_exact(name, got[~nan], ref[~nan])


@pytest.mark.parametrize("Wn", [2, 5, 16, 33, 1024])
def test_server_exact_sum_boundary(Wn):
    """The regrouped (table) sum is taken only where it equals the ordered fp64 sum:
    every output matches the oracle's ordered sum at, just beyond and far beyond the
    exactness bound, and with non-finite scales."""
    sizes = [4096, 2048 * 3 + 5, 31, 4096 + 64, 8192, 2053, 4096, 999]
    off = W.offsets_from_sizes(sizes)
    buf = CompressBuffers(off)
    n, words, nch = buf.n, buf.words, buf.n_chunks
    rng = np.random.default_rng(1700 + Wn)
    wb = rng.integers(0, 1 << 32, size=(Wn, words), dtype=np.uint64).astype(np.uint32)
    sc = np.stack(_boundary_cases(rng, Wn), axis=1)  # [Wn, nch]
    assert sc.shape == (Wn, nch)
    es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    say(f"server exact-sum boundary W={Wn}")
    wbd = torch.from_numpy(wb.view(np.int32).copy()).to(DEV)
    scd = torch.from_numpy(sc.copy()).to(DEV)
    esd = torch.from_numpy(es.copy()).to(DEV)
    sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
    sscales = torch.zeros(nch, dtype=torch.float32, device=DEV)
    md = torch.zeros(n, dtype=torch.float32, device=DEV)
    ob.onebit_server_reduce(buf.plan, wbd, scd, esd, sbits, sscales, md, buf.ws)
    rb, rs, m_out = oracle.server_reduce(off, wb, sc, es)
    torch.cuda.synchronize()
    assert_bits_exact("server bits", host(sbits).view(np.uint32), rb)
    _assert_same_or_both_nan("server scales", host(sscales), rs)
    _assert_same_or_both_nan("server e", host(esd), es)
    _assert_same_or_both_nan("server m", host(md), m_out)


def test_server_exact_sum_boundary_on_a_two_pass_chunk():
    """The same boundary cases with the first chunk too large for the one-pass kernel,
    so that its server tiles take the two-pass kernels (W = 16)."""
    Wn = 16
    big = max(ob.onebit_onepass_max_elements(), 1) + 4097
    off = W.offsets_from_sizes([big, 2048 * 3 + 5, 31, 4096 + 64, 8192, 2053, 4096, 999])
    buf = CompressBuffers(off)
    n, words, nch = buf.n, buf.words, buf.n_chunks
    rng = np.random.default_rng(2900)
    wb = rng.integers(0, 1 << 32, size=(Wn, words), dtype=np.uint64).astype(np.uint32)
    cases = _boundary_cases(rng, Wn)
    for first in (0, 2):                       # the widest exact spread, then one where the orders differ
        order = [first] + list(range(1, nch))
        sc = np.stack([cases[k] for k in order], axis=1)
        assert sc.shape == (Wn, nch)
        es = (rng.standard_normal(n) * 1e-5).astype(np.float32)
        say(f"server two-pass boundary, first chunk case {first}")
        wbd = torch.from_numpy(wb.view(np.int32).copy()).to(DEV)
        scd = torch.from_numpy(sc.copy()).to(DEV)
        esd = torch.from_numpy(es.copy()).to(DEV)
        sbits = torch.zeros(words, dtype=torch.int32, device=DEV)
        sscales = torch.zeros(nch, dtype=torch.float32, device=DEV)
        md = torch.zeros(n, dtype=torch.float32, device=DEV)
        ob.onebit_server_reduce(buf.plan, wbd, scd, esd, sbits, sscales, md, buf.ws)
        rb, rs, m_out = oracle.server_reduce(off, wb, sc, es)
        torch.cuda.synchronize()
        assert_bits_exact("server bits", host(sbits).view(np.uint32), rb)
        _assert_same_or_both_nan("server scales", host(sscales), rs)
        _assert_same_or_both_nan("server e", host(esd), es)
        _assert_same_or_both_nan("server m", host(md), m_out)
        assert ob.onebit_workspace_status(buf.ws) == 0

"""GPU parity of the QSGD gradient quantizer and of the W-worker decode/average
against the oracle (codes, norms and decoded values bit for bit).

Small cases cover the 1024-element fast path and the generic path (bucket sizes
2, 30, 64, 1000, 4096), ragged last buckets, odd n (4-bit pad nibble), fp32 /
bf16 / fp16 gradients, zero and single-value buckets, signed zeros, buckets whose
ratios are exact levels, and a wide dynamic range.  The reduce covers W = 1, 2,
3, 8, buckets that are and are not multiples of 8, n not a multiple of 8, fp32
and bf16 outputs, padded worker rows, and arbitrary codes with norms over the whole
binary32 range (W = 1, 5, 16, 33).  Full size: the 1.3e9-parameter gradient of
8 workers, bucket 1024, sampled buckets of every worker and sampled buckets of two
shards' averages (the first and the ragged last).
"""
import numpy as np
import pytest
import torch

import oracle
from error_compensated_bit_amd import onebit as ob
from error_compensated_bit_amd import workloads as W
from gpu_helpers import DEV, host
from parity import assert_exact, check_bf16, say

pytestmark = pytest.mark.gpu


def code_bytes(n, bits):
    return (n + 1) // 2 if bits == 4 else n


def special_gradient(n, rng):
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 2, n)).astype(np.float32)
    if n >= 4096:
        g[0:64] = 0.0                                      # zero bucket for buckets <= 64
        g[64:128] = 0.0
        g[100] = -889 / 16                                 # lone value
        g[128:192] = np.tile(np.array([0.0, -0.0], np.float32), 32)
        g[256:320] = 0.0
        g[256:259] = [2.0, -3.0, 6.0]                      # |.| = 7: exact 4-bit levels
        g[1024:2048] *= 1e-30                              # tiny bucket
    return g


def to_device(g, dt):
    t = torch.from_numpy(g).to(DEV)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
        return t, host(t)
    if dt == "f16":
        t = t.to(torch.float16)
        return t, t.cpu().numpy()
    return t, g


@pytest.mark.parametrize("bucket", [1024, 2, 30, 64, 1000, 4096])
@pytest.mark.parametrize("bits", [4, 8])
def test_quantize_parity(bucket, bits):
    for dt in ("f32", "bf16", "f16"):
        for n in (1, 2 * bucket + 7, 9 * 1024 + 333, 4 * 1024):    # 4096: no ragged bucket at 1024
            if bits == 4 and n % 2 == 1 and n > 1:
                pass                                       # odd n: pad nibble
            rng = np.random.default_rng(n * 7 + bucket + bits)
            g = special_gradient(n, rng)
            if dt == "f16":
                g = np.clip(g, -6e4, 6e4)
            gd, gh = to_device(g, dt)
            nb = (n + bucket - 1) // bucket
            codes = torch.full((code_bytes(n, bits) + 16,), 0xAB, dtype=torch.uint8, device=DEV)
            norms = torch.zeros(nb, device=DEV)
            seed = 1234 + n
            ob.qsgd_quantize(gd, bucket, bits, seed, codes, norms)
            rc, rn = oracle.qsgd_quantize(gh, bucket=bucket, bits=bits, seed=seed)
            torch.cuda.synchronize()
            tag = f"bucket {bucket} bits {bits} {dt} n {n}"
            assert_exact(f"{tag} norms", host(norms), rn)
            got = host(codes)
            assert_exact(f"{tag} codes", got[:rc.size], rc)
            assert np.all(got[rc.size:] == 0xAB), f"{tag}: wrote past the codes"
            y = torch.zeros(n, device=DEV)
            ob.qsgd_reduce(codes, norms, n, bucket, bits, out_f32=y)
            ry, _ = oracle.qsgd_reduce(rc, rn, n, bucket=bucket, bits=bits)
            torch.cuda.synchronize()
            assert_exact(f"{tag} decoded", host(y), ry)
    say(f"  qsgd quantize bucket {bucket} bits {bits}: fp32 / bf16 / fp16 match")


def extreme_f32(n, rng):
    """fp32 gradients over the whole exponent range below 2^61 (subnormals and signed
    zeros included), with a bucket of subnormals only and one spanning 2^-120 .. 2^60."""
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    e = (u >> 23) & 0xFF
    big = e > 187
    u[big] = (u[big] & 0x807FFFFF) | (rng.integers(0, 188, int(big.sum())).astype(np.uint32) << 23)
    u[2048:3072] &= 0x807FFFFF                                       # subnormal bucket
    ex = rng.integers(7, 188, 1024).astype(np.uint32)
    u[4096:5120] = (u[4096:5120] & 0x807FFFFF) | (ex << 23)
    return u.view(np.float32)


@pytest.mark.parametrize("bucket", [1024, 1000])
@pytest.mark.parametrize("bits", [4, 8])
def test_extreme_exponents(bucket, bits):
    """|g| / norm is formed from one fp64 reciprocal of the norm per bucket; it must
    round exactly as the oracle's fp32 division, subnormal quotients included."""
    for dt in ("f32", "bf16"):
        n = 8 * 1024 + 77
        g = extreme_f32(n, np.random.default_rng(bucket + bits))
        gd, gh = to_device(g, dt)
        nb = (n + bucket - 1) // bucket
        codes = torch.zeros(code_bytes(n, bits), dtype=torch.uint8, device=DEV)
        norms = torch.zeros(nb, device=DEV)
        ob.qsgd_quantize(gd, bucket, bits, 31, codes, norms)
        rc, rn = oracle.qsgd_quantize(gh, bucket=bucket, bits=bits, seed=31)
        torch.cuda.synchronize()
        tag = f"extreme bucket {bucket} bits {bits} {dt}"
        say(tag)
        assert_exact(f"{tag} norms", host(norms), rn)
        assert_exact(f"{tag} codes", host(codes), rc)


@pytest.mark.parametrize("workers", [1, 2, 3, 8])
@pytest.mark.parametrize("bucket,bits", [(1024, 4), (1000, 8), (30, 4), (2, 8), (4096, 4)])
@pytest.mark.parametrize("n", [3 * 4096 + 13, 16 * 1000 + 7, 16 * 63 + 5])
def test_reduce_parity(workers, bucket, bits, n):
    """n: whole waves of 64 x 16 elements plus a ragged tail, then a partly filled
    last wave (1000 and 63 groups of 16) plus a tail."""
    nb = (n + bucket - 1) // bucket
    stride = (code_bytes(n, bits) + 15) // 16 * 16 + 32      # padded worker rows
    codes = torch.zeros((workers, stride), dtype=torch.uint8, device=DEV)
    norms = torch.zeros((workers, nb + 3), device=DEV)
    rcs, rns = [], []
    for w in range(workers):
        g = (np.random.default_rng(50 + w).standard_normal(n) * 10.0 ** (-w % 4)).astype(np.float32)
        gd = torch.from_numpy(g).to(DEV).to(torch.bfloat16)
        ob.qsgd_quantize(gd, bucket, bits, 99 + w, codes[w], norms[w])
        rc, rn = oracle.qsgd_quantize(host(gd), bucket=bucket, bits=bits, seed=99 + w)
        rcs.append(np.pad(rc, (0, stride - rc.size)))
        rns.append(np.pad(rn, (0, 3)))
    y = torch.zeros(n, device=DEV)
    yb = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    ob.qsgd_reduce(codes, norms, n, bucket, bits, out_f32=y, out_bf16=yb)
    ry, ryb = oracle.qsgd_reduce(np.stack(rcs), np.stack(rns), n, bucket=bucket, bits=bits, want_bf16=True)
    torch.cuda.synchronize()
    tag = f"W={workers} bucket {bucket} bits {bits} n {n}"
    assert_exact(f"{tag} codes", host(codes), np.stack(rcs))
    assert_exact(f"{tag} mean", host(y), ry)
    check_bf16(f"{tag} mean bf16", host(yb), ryb)


@pytest.mark.parametrize("workers", [1, 5, 16, 33])
@pytest.mark.parametrize("bucket,bits", [(1024, 4), (1024, 8), (30, 4), (16, 8)])
def test_reduce_arbitrary_codes_and_norms(workers, bucket, bits):
    """Every byte pattern is a valid code (pair); norms span the finite binary32
    range, subnormals included, with up to 60 binary orders between workers of a
    bucket: the decode is the fp64 sum of exact level * norm products, one division
    by s * W, one rounding.  A last run makes one worker's norm of one bucket
    infinite: +-inf where every worker's level there is non-zero with one sign, NaN
    where the sum meets opposite infinities or a level 0 meets the infinite norm."""
    rng = np.random.default_rng(7 * workers + bits + bucket)
    n = 5 * 1024 + 16 * 37 + 9
    nb = (n + bucket - 1) // bucket
    cb = code_bytes(n, bits)
    stride = (cb + 15) // 16 * 16
    c = rng.integers(0, 256, (workers, stride), dtype=np.uint8)
    if bits == 4:
        c[:, cb - 1] &= 0x0F                               # pad nibble of the odd tail
    c[:, cb:] = 0
    base = rng.integers(-150, 67, nb)
    e = base[None, :] + rng.integers(0, 61, (workers, nb))       # norms below 2^127
    nm = np.ldexp(rng.uniform(1.0, 2.0, (workers, nb)), e).astype(np.float32)
    nm[:, 1] = 0.0                                         # a zero bucket
    codes = torch.from_numpy(c).to(DEV)
    norms = torch.from_numpy(nm).to(DEV)
    y = torch.zeros(n, device=DEV)
    yb = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    ob.qsgd_reduce(codes, norms, n, bucket, bits, out_f32=y, out_bf16=yb)
    ry, ryb = oracle.qsgd_reduce(c, nm, n, bucket=bucket, bits=bits, want_bf16=True)
    torch.cuda.synchronize()
    tag = f"arbitrary codes W={workers} bucket {bucket} bits {bits}"
    say(tag)
    assert np.all(np.isfinite(nm))
    assert_exact(f"{tag} mean", host(y), ry)
    check_bf16(f"{tag} mean bf16", host(yb), ryb)
    nm[workers // 2, 2] = np.inf
    norms.copy_(torch.from_numpy(nm))
    ob.qsgd_reduce(codes, norms, n, bucket, bits, out_f32=y)
    ry, _ = oracle.qsgd_reduce(c, nm, n, bucket=bucket, bits=bits)
    torch.cuda.synchronize()
    got = host(y)
    nan = np.isnan(ry)
    assert np.array_equal(np.isnan(got), nan), f"{tag} infinite norm: NaN positions differ"
    assert_exact(f"{tag} infinite norm, non-NaN values", got[~nan], ry[~nan])
    assert np.isinf(ry).any() or nan.any()


def test_argument_errors():
    g = torch.zeros(64, device=DEV)
    codes = torch.zeros(64, dtype=torch.uint8, device=DEV)
    norms = torch.zeros(4, device=DEV)
    for kw in (dict(bucket=3, bits=4), dict(bucket=16, bits=6), dict(bucket=0, bits=8)):
        with pytest.raises(ob.OnebitError) as ei:
            ob.qsgd_quantize(g, kw["bucket"], kw["bits"], 0, codes, norms)
        assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError) as ei:
        ob.qsgd_quantize(g[1:], 16, 8, 0, codes, norms)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN
    with pytest.raises(ob.OnebitError) as ei:
        ob.qsgd_reduce(codes, norms, 64, 16, 8)                        # no output
    assert ei.value.status == ob.ONEBIT_ERR_INVALID
    rows = torch.zeros((2, 72), dtype=torch.uint8, device=DEV)
    with pytest.raises(ob.OnebitError) as ei:                          # row stride not a multiple of 16
        ob.qsgd_reduce(rows, torch.zeros((2, 4), device=DEV), 64, 16, 8, out_f32=torch.zeros(64, device=DEV))
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN


@pytest.mark.parametrize("bits", [4, 8])
def test_full_size_eight_workers(bits):
    q = W.QsgdWorkload()
    n, bucket, nb = q.n, q.bucket, (q.n + q.bucket - 1) // q.bucket
    cb = code_bytes(n, bits)
    stride = (cb + 15) // 16 * 16
    codes = torch.zeros((q.W, stride), dtype=torch.uint8, device=DEV)
    norms = torch.zeros((q.W, nb), device=DEV)
    per = 2 if bits == 4 else 1
    sample_b = sorted({0, nb - 1, nb - 2} | set(int(b) for b in np.random.default_rng(bits).choice(nb, 29, replace=False)))
    keep = {}
    for w in range(q.W):
        gd = W.qsgd_gradient(q, w, device=DEV)
        seed = 7000 + w
        ob.qsgd_quantize(gd, bucket, bits, seed, codes[w], norms[w])
        torch.cuda.synchronize()
        for b in sample_b:
            lo, hi = b * bucket, min((b + 1) * bucket, n)
            gs = host(gd[lo:hi])
            rc, rn = oracle.qsgd_quantize(gs, bucket=bucket, bits=bits, seed=seed, first_index=lo)
            assert_exact(f"worker {w} bucket {b} codes", host(codes[w, lo // per:(hi + per - 1) // per]), rc)
            assert_exact(f"worker {w} bucket {b} norm", host(norms[w, b:b + 1]), rn)
        del gd
        say(f"  qsgd{bits} worker {w}: {len(sample_b)} buckets match")
    for s in (0, q.W - 1):
        lo = s * q.shard
        hi = min(lo + q.shard, n)
        m = hi - lo
        y = torch.zeros(m, device=DEV)
        ob.qsgd_reduce(codes[:, lo // per:], norms[:, lo // bucket:], m, bucket, bits, out_f32=y)
        torch.cuda.synchronize()
        sb = (m + bucket - 1) // bucket
        for b in sorted({0, sb - 1} | set(int(x) for x in np.random.default_rng(s).choice(sb, 14, replace=False))):
            blo, bhi = b * bucket, min((b + 1) * bucket, m)
            gb = (lo + blo) // bucket
            rc = np.stack([host(codes[w, (lo + blo) // per:(lo + bhi + per - 1) // per]) for w in range(q.W)])
            rn = np.stack([host(norms[w, gb:gb + 1]) for w in range(q.W)])
            ry, _ = oracle.qsgd_reduce(rc, rn, bhi - blo, bucket=bucket, bits=bits)
            assert_exact(f"shard {s} bucket {b} mean", host(y[blo:bhi]), ry)
        say(f"  qsgd{bits} shard {s} ({m} elements): sampled buckets match")


@pytest.mark.parametrize("bucket,bits", [(1024, 4), (1024, 8), (30, 4), (1000, 8)])
@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9])
@pytest.mark.parametrize("n", [5 * 1024 + 77, 3 * 1024, 500])
def test_loco_parity(bucket, bits, beta, n):
    rng = np.random.default_rng(bucket + bits)
    e0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    for dt in ("f32", "bf16"):
        ed = torch.from_numpy(e0.copy()).to(DEV)
        er = e0.copy()
        codes = torch.zeros(code_bytes(n, bits), dtype=torch.uint8, device=DEV)
        norms = torch.zeros((n + bucket - 1) // bucket, device=DEV)
        for step in range(3):
            g = (np.random.default_rng(step).standard_normal(n) * 10.0 ** -(2 + step)).astype(np.float32)
            gd, gh = to_device(g, dt)
            ob.loco_quantize(gd, ed, bucket, bits, beta, 500 + step, codes, norms)
            rc, rn = oracle.loco_quantize(gh, er, bucket=bucket, bits=bits, beta=beta, seed=500 + step)
            torch.cuda.synchronize()
            tag = f"loco bucket {bucket} bits {bits} beta {beta} {dt} step {step}"
            assert_exact(f"{tag} codes", host(codes), rc)
            assert_exact(f"{tag} norms", host(norms), rn)
            assert_exact(f"{tag} err_avg", host(ed), er)


@pytest.mark.parametrize("n", [1023, 1024, 1025, 2048, 2049])
@pytest.mark.parametrize("bits", [4, 8])
def test_bucket_1024_whole_and_last(n, bits):
    """Buckets of 1024 go to two kernels (whole buckets, then a ragged last one):
    sizes with only a last bucket, only whole ones, and both; plain and LoCo."""
    rng = np.random.default_rng(n + bits)
    for dt in ("f32", "bf16", "f16"):
        g = special_gradient(n, rng)
        if dt == "f16":
            g = np.clip(g, -6e4, 6e4)
        gd, gh = to_device(g, dt)
        nb = (n + 1023) // 1024
        codes = torch.full((code_bytes(n, bits) + 16,), 0xAB, dtype=torch.uint8, device=DEV)
        norms = torch.zeros(nb, device=DEV)
        ob.qsgd_quantize(gd, 1024, bits, 77 + n, codes, norms)
        rc, rn = oracle.qsgd_quantize(gh, bucket=1024, bits=bits, seed=77 + n)
        torch.cuda.synchronize()
        tag = f"n {n} bits {bits} {dt}"
        assert_exact(f"{tag} codes", host(codes)[:rc.size], rc)
        assert (host(codes)[rc.size:] == 0xAB).all(), f"{tag}: bytes past the codes written"
        assert_exact(f"{tag} norms", host(norms), rn)
        e0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        ed, er = torch.from_numpy(e0.copy()).to(DEV), e0.copy()
        ob.loco_quantize(gd, ed, 1024, bits, 0.5, 91 + n, codes, norms)
        rc, rn = oracle.loco_quantize(gh, er, bucket=1024, bits=bits, beta=0.5, seed=91 + n)
        torch.cuda.synchronize()
        assert_exact(f"{tag} loco codes", host(codes)[:rc.size], rc)
        assert_exact(f"{tag} loco norms", host(norms), rn)
        assert_exact(f"{tag} loco err_avg", host(ed), er)


def test_loco_argument_errors():
    g = torch.zeros(64, device=DEV)
    e = torch.zeros(64, device=DEV)
    codes = torch.zeros(64, dtype=torch.uint8, device=DEV)
    norms = torch.zeros(4, device=DEV)
    for beta in (-0.1, 1.5, float("nan")):
        with pytest.raises(ob.OnebitError) as ei:
            ob.loco_quantize(g, e, 16, 8, beta, 0, codes, norms)
        assert ei.value.status == ob.ONEBIT_ERR_INVALID
    with pytest.raises(ob.OnebitError) as ei:
        ob.loco_quantize(g, e[1:], 16, 8, 0.5, 0, codes, norms)
    assert ei.value.status == ob.ONEBIT_ERR_ALIGN


def test_loco_full_size_two_steps():
    q = W.QsgdWorkload()
    n, bucket, bits = q.n, q.bucket, 4
    nb = (n + bucket - 1) // bucket
    e = torch.zeros(n, device=DEV)
    codes = torch.zeros(code_bytes(n, bits), dtype=torch.uint8, device=DEV)
    norms = torch.zeros(nb, device=DEV)
    sample_b = sorted({0, nb - 1} | set(int(b) for b in np.random.default_rng(9).choice(nb, 30, replace=False)))
    for step in range(2):
        gd = W.qsgd_gradient(q, step, device=DEV)
        before = {b: (host(gd[b * bucket:min((b + 1) * bucket, n)]), host(e[b * bucket:min((b + 1) * bucket, n)]))
                  for b in sample_b}
        ob.loco_quantize(gd, e, bucket, bits, 0.9, 900 + step, codes, norms)
        torch.cuda.synchronize()
        for b in sample_b:
            lo, hi = b * bucket, min((b + 1) * bucket, n)
            gs, es = before[b]
            rc, rn = oracle.loco_quantize(gs, es, bucket=bucket, bits=bits, beta=0.9, seed=900 + step, first_index=lo)
            assert_exact(f"step {step} bucket {b} codes", host(codes[lo // 2:(hi + 1) // 2]), rc)
            assert_exact(f"step {step} bucket {b} norm", host(norms[b:b + 1]), rn)
            assert_exact(f"step {step} bucket {b} err_avg", host(e[lo:hi]), es)
        del gd
        say(f"  loco step {step}: {len(sample_b)} buckets match")


# (a, b) with a^2 + b^2 = m^2 and m odd just above 2^24: m lies exactly halfway
# between the fp32 values m - 1 and m + 1, so the bucket norm is a rounding tie (to
# the even one, m - 1) and the quantizer must take its compensated sum.
NORM_TIES = [(16777215, 8192, 16777217), (16777207, 24576, 16777225), (8470365, 14482028, 16777253)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("loco", [False, True])
def test_norm_ties_take_the_compensated_sum(bits, loco):
    """Buckets whose norm is an exact fp32 rounding tie (whole buckets of 1024 and the
    ragged last one, several binades), next to ordinary buckets: norms, codes (and the
    LoCo error average) equal the oracle's, and the norms are the tie's even value."""
    n = 6 * 1024 + 300
    rng = np.random.default_rng(4400 + bits + 10 * loco)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    want = {}
    for b, (scale, (a_, b_, m)) in enumerate(zip([2.0 ** -30, 2.0 ** -90, 2.0 ** 40, 2.0 ** -12, 1.0, 2.0 ** -40],
                                                 NORM_TIES * 2)):
        if b == 4:
            continue                                       # an ordinary bucket
        lo = 1024 * b
        g[lo:lo + 1024] = 0.0
        g[lo + 7] = np.float32(a_ * scale)
        g[lo + 900] = np.float32(-b_ * scale)
        want[b] = np.float32((m - 1) * scale)
    tail = 6 * 1024
    g[tail:] = 0.0
    g[tail + 5], g[tail + 299] = np.float32(NORM_TIES[0][0] * 2.0 ** -20), np.float32(NORM_TIES[0][1] * 2.0 ** -20)
    want[6] = np.float32((NORM_TIES[0][2] - 1) * 2.0 ** -20)
    gd = torch.from_numpy(g).to(DEV)
    nb = 7
    codes = torch.zeros(code_bytes(n, bits), dtype=torch.uint8, device=DEV)
    norms = torch.zeros(nb, device=DEV)
    if loco:
        err = np.zeros(n, np.float32)
        errd = torch.from_numpy(err.copy()).to(DEV)
        ob.loco_quantize(gd, errd, 1024, bits, 0.9, 77, codes, norms)
        rc, rn = oracle.loco_quantize(g, err, bucket=1024, bits=bits, beta=0.9, seed=77)
    else:
        ob.qsgd_quantize(gd, 1024, bits, 77, codes, norms)
        rc, rn = oracle.qsgd_quantize(g, bucket=1024, bits=bits, seed=77)
    torch.cuda.synchronize()
    for b, v in want.items():
        assert rn[b] == v, (b, rn[b], v)                    # the oracle's norm is the tie's even value
    tag = f"norm ties bits {bits} loco {loco}"
    say(tag)
    assert_exact(f"{tag} norms", host(norms), rn)
    assert_exact(f"{tag} codes", host(codes), rc)
    if loco:
        assert_exact(f"{tag} error average", host(errd), err)

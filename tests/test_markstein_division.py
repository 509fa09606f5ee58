"""The QSGD decode divides an fp64 sum by s * W (s = 7 or 127 levels, W workers)
without an fp64 division instruction sequence: with r = RN64(1 / (s W)) formed on
the host, q = RN(a r), res = fma(-q, s W, a) (exact), q' = fma(res, r, q).  By
Markstein's theorem (Markstein 1990; Muller et al., Handbook of Floating-Point
Arithmetic, the section on division with a fused multiply-add) q' is the correctly
rounded quotient when q is within one ulp of it and r is the correctly rounded
reciprocal.  tests/markstein_check.c checks that against IEEE division for every
divisor s W with W <= 1024, on decode-shaped sums, on arbitrary fp64 dividends, on
quotients next to fp64 halfway points and on infinite and NaN dividends (for which
the residual is NaN and q itself is returned); built without the correction step it
must find mismatches."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def _run(extra):
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "mk")
        subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", *extra, "-o", exe,
                        os.path.join(HERE, "markstein_check.c"), "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    return int(out[-2]), int(out[-1])


def test_corrected_quotient_is_ieee_division():
    cases, bad = _run([])
    assert cases == 2 * 1024 * 3000 + 3 * 1024 and bad == 0


def test_check_finds_the_uncorrected_quotient():
    _, bad = _run(["-DUNCORRECTED"])
    assert bad > 1000

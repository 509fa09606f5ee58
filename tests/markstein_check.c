/* Brute-force check of the fp64 quotient RN(a / d) formed, with r = RN(1 / d), as
 *   q = RN(a * r);  res = RN(a - d * q) (one fused multiply-add, exact);
 *   q' = RN(q + res * r) (one fused multiply-add)
 * against IEEE division, for the divisors d = s * W of the QSGD decode
 * (s = 7 or 127 levels, W = 1 ... 1024 workers) and dividends a that are the
 * decode's fp64 sums of level * norm products, random fp64 numbers, and values
 * whose quotient lies next to a point halfway between two fp64 numbers.
 * Markstein's theorem (q within one ulp of a / d, r the correctly rounded
 * reciprocal, no underflow or overflow) says q' is the correctly rounded quotient.
 * Prints the number of cases and of mismatches.  Built with -DUNCORRECTED it
 * returns q itself, which must mismatch (the check's own sanity test). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}

static double corrected(double a, double d, double r)
{
    const double q = a * r;
#ifdef UNCORRECTED
    (void)d;
    return q;
#else
    const double res = fma(-q, d, a);
    return isfinite(res) ? fma(res, r, q) : q;
#endif
}

int main(void)
{
    long cases = 0, bad = 0;
    for (int si = 0; si < 2; ++si) {
        const int s = si ? 127 : 7;
        for (int W = 1; W <= 1024; ++W) {
            const double d = (double)s * (double)W;
            const double r = 1.0 / d;
            for (int k = 0; k < 3000; ++k) {
                double a;
                const int kind = k % 3;
                if (kind == 0) {            /* sum of W exact level * norm products */
                    a = 0.0;
                    const int e0 = (int)(next() % 300) - 160;
                    const int terms = W < 32 ? W : 32;
                    for (int w = 0; w < terms; ++w) {
                        const double lv = (double)(next() % (uint64_t)(s + 1));
                        const double nm = ldexp((double)((next() & 0xFFFFFFu) | 0x800000u), e0 - 23 + (int)(next() % 19));
                        a += (next() & 1) ? -lv * nm : lv * nm;
                    }
                } else if (kind == 1) {     /* any fp64 number */
                    const uint64_t m = (next() & 0xFFFFFFFFFFFFFull) | 0x10000000000000ull;
                    a = ldexp((double)m, (int)(next() % 600) - 352);
                    if (next() & 1) a = -a;
                } else {                    /* quotient next to an fp64 halfway point */
                    const uint64_t m = (next() & 0xFFFFFFFFFFFFFull) | 0x10000000000000ull;
                    const long double qm = ((long double)m + 0.5L) * ldexpl(1.0L, (int)(next() % 200) - 152);
                    a = (double)(qm * (long double)d);
                }
                const double ref = a / d;
                const double got = corrected(a, d, r);
                ++cases;
                if (memcmp(&ref, &got, sizeof ref) != 0) {
                    if (bad < 5) printf("mismatch a=%a d=%g ref=%a got=%a\n", a, d, ref, got);
                    ++bad;
                }
            }
        }
    }
    /* infinite and NaN dividends: the quotient is the dividend's infinity or a NaN */
    const double special[3] = {INFINITY, -INFINITY, NAN};
    for (int k = 0; k < 3; ++k)
        for (int W = 1; W <= 1024; ++W) {
            const double d = 127.0 * W, r = 1.0 / d;
            const double ref = special[k] / d, got = corrected(special[k], d, r);
            ++cases;
            if (!(isnan(ref) ? isnan(got) : ref == got)) ++bad;
        }
    printf("%ld %ld\n", cases, bad);
    return 0;
}

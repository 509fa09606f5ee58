// quant_common.h -- arithmetic shared by the stochastic quantizers (qsdp.hip,
// qsgd.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace onebit {

// fl32(a / b) for fp32 a, b, given rb = RN64(1 / b) (one fp64 division per bucket).
// The fp64 product a * rb is within 3 * 2^-53 (relative) of a / b.  A quotient of two
// 24-bit numbers that is not itself an fp32 number lies more than 2^-49 (relative)
// from every point halfway between two consecutive fp32 numbers: a - b * m is a
// non-zero multiple of ulp(b) * ulp(a / b) / 2 for such a point m.  So no halfway
// point separates the product from the quotient, and rounding the product to fp32
// gives the correctly rounded quotient, subnormal, infinite and NaN cases included.
// This is the argument that makes double rounding harmless for division whenever the
// wider format has at least 2p + 2 bits (here 53 >= 2 * 24 + 2).  It replaces the
// ten-instruction fp32 division sequence by three instructions per element.
__device__ __forceinline__ double recip_rn64(float b) { return __ddiv_rn(1.0, (double)b); }

__device__ __forceinline__ float div_by_recip(float a, double rb) { return (float)__dmul_rn((double)a, rb); }

// RN64(a / d) for fp64 a and finite d > 0, given rd = RN64(1 / d), with one product
// and two fused multiply-adds instead of the fp64 division sequence: q = RN(a rd) is
// within one ulp of a / d, the residual a - d q is exact in one fma, and q + res rd
// rounded once is the correctly rounded quotient (Markstein's theorem; no fp64
// underflow or overflow can occur for the decode's finite operands).  An infinite
// or NaN a gives a NaN residual; q itself (+-inf or NaN) is then the quotient.
__device__ __forceinline__ double div_rn64(double a, double d, double rd) {
    const double q = __dmul_rn(a, rd);
    const double res = __fma_rn(-q, d, a);
    return __builtin_isfinite(res) ? __fma_rn(res, rd, q) : q;
}

}  // namespace onebit

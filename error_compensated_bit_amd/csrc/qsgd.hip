// qsgd.hip -- the gradient side of QSDP: the standard unbiased gradient
// compressor (QSDP review, "proposed method", naming Alistarh et al. 2017; QSGD,
// sec. 3.1) and the decode-and-average of W workers' streams that the shard
// owner of a quantized reduce-scatter performs.  The LoCo variant (LoCo summary,
// method details) quantizes g + err, where err is a moving average of past
// compression errors, and updates that average in the same pass.
//
// Per bucket of the gradient: norm = ||g||_2 (fp64 double-double sum of squares,
// fp64 square root, one rounding to fp32); s = 2^(bits-1) - 1 levels of |g|/norm,
// rounded up at random with probability equal to the fractional part, so the
// decoded value norm * level / s carries the sign of g and has expectation g.
// Decoding rounds that real value once: the product level * norm is exact in fp64,
// W workers' products are summed in fp64 in worker order, divided once by s * W
// (correctly rounded) and rounded once to fp32.
// Codes: sign bit on top, level below; 4-bit codes two per byte (even element
// low).  Random words: Philox4x32-10 keyed by the seed, counter = element index
// / 4, word = element index % 4 -- the weights' layout; the caller gives the
// gradient stream its own seed.
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "quant_common.h"

namespace onebit {

struct GArgs {
    const void *g;
    float *err;          // LoCo: moving average of the compression error, in place
    float beta, obeta;   // LoCo: its weights beta and 1 - beta
    int64_t n;
    int64_t n_buckets;
    int32_t bucket;
    uint32_t k0, k1;
    uint8_t *codes;
    float *norms;
};

template <int GT>
__device__ __forceinline__ float load_grad(const void *g, int64_t i) {
    if (GT == kGradF32) return static_cast<const float *>(g)[i];
    return half_bits_to_float<GT>(static_cast<const uint16_t *>(g)[i]);
}

// Level and sign of one element, given its uniform word; rnorm = RN64(1 / norm).
template <int BITS>
__device__ __forceinline__ uint32_t qsgd_code(float g, float norm, double rnorm, uint32_t u) {
    constexpr float S = (float)((1 << (BITS - 1)) - 1);
    if (norm == 0.0f) return 0u;
    const float t = div_by_recip(fabsf(g), rnorm);       // = fl32(|g| / norm) <= 1: norm >= |g|
    const float v = mul_rn(t, S);
    const float l = floorf(v);
    const float p = sub_rn(v, l);                          // exact, in [0, 1)
    const uint32_t thr = (uint32_t)ldexpf(p, 32);          // floor(p * 2^32), exact
    const uint32_t level = (uint32_t)l + (u < thr ? 1u : 0u);
    return (g < 0.0f ? (1u << (BITS - 1)) : 0u) | level;
}

// The decoded value of one code, times s, added to acc: +-level * norm is exact in
// fp64 (at most 7 + 24 significant bits), so one fused multiply-add is the fp64 sum
// of the exact product.  The code sits at bit P of the 32-bit word w; its sign bit
// goes straight into the sign of the converted level (the level's own sign bit is 0).
template <int BITS, int P>
__device__ __forceinline__ double qsgd_accumulate(double acc, uint32_t w, double norm) {
    constexpr uint32_t S = (1u << (BITS - 1)) - 1u;
    constexpr uint32_t SIGN = 1u << (P + BITS - 1);
    const double lv = (double)((w >> P) & S);
    const uint32_t hi = (uint32_t)(__double_as_longlong(lv) >> 32) | ((w & SIGN) << (32 - BITS - P));
    const double slv = __hiloint2double((int)hi, (int)(uint32_t)__double_as_longlong(lv));
    return __fma_rn(slv, norm, acc);
}

// LoCo: the new moving average of the compression error, from the old one, the
// compensated value h, its code and the bucket's norm.  The decode is the W = 1
// average: fl32((0 + +-level * norm) / s).
template <int BITS>
__device__ __forceinline__ float loco_update(const GArgs &a, float ea, float h, uint32_t code, float norm) {
    constexpr double S = (double)((1u << (BITS - 1)) - 1u);
    constexpr double RS = 1.0 / S;   // correctly rounded at compile time
    const float y = (float)div_rn64(qsgd_accumulate<BITS, 0>(0.0, code, (double)norm), S, RS);
    const float err = sub_rn(h, y);
    return add_rn(mul_rn(a.beta, ea), mul_rn(a.obeta, err));
}

__device__ __forceinline__ float norm_of(DD acc) {
    const DD t = wave_sum_dd(acc);
    return (float)__dsqrt_rn(t.hi);
}

// The bucket norm fl32(sqrt(S)) from a plain fp64 sum S' of the (exact) squares,
// where that is provably the value the compensated sum gives.  All terms are
// non-negative, so in any order |S' - S| <= (n - 1) 2^-53 S < 2^-43 S for n <= 1024,
// and sqrt(S') is within 2^-44 of sqrt(S), relatively; the compensated sum is within
// 2^-52 of S.  Where sqrt(S') lies farther than 2^-40 of itself from the midpoint
// between the two fp32 values around it, all of them round to the same fp32 value.
// The butterfly sum leaves the same bits in every lane (each step adds the same two
// values, in either order), so the answer is the same over the wave.  Returns false
// (the caller takes the compensated sum) near a midpoint, about once in 2^16
// buckets, for a non-finite sum and at the top of the fp32 range.  Each lane passes
// the plain sum of its own squares.
__device__ __forceinline__ bool norm_from_plain_sum(double s, float &norm) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s = __dadd_rn(s, __shfl_xor(s, o));
    const double r = __dsqrt_rn(s);
    if (r == 0.0) {
        norm = 0.0f;
        return true;
    }
    const float f = (float)r;
    const uint32_t fb = __float_as_uint(f);
    const float nb = __uint_as_float((double)f <= r ? fb + 1u : fb - 1u);   // the neighbour on r's side
    if (!isfinite(r) || !isfinite(f) || !isfinite(nb)) return false;
    const double mid = 0.5 * ((double)f + (double)nb);                        // exact
    if (!(fabs(r - mid) > 0x1p-40 * r)) return false;
    norm = f;
    return true;
}

// Group j (four elements) of this lane's sixteen in a whole bucket staged in LDS:
// the value that is quantized (g, or with LoCo h = g + err) and, with LoCo, err.
template <int GT, bool LOCO>
__device__ __forceinline__ void staged_group(const float4 *wg, const float4 *we, int lane, int j, float (&h)[4],
                                             float (&e)[4]) {
    if (GT == kGradF32) {
        const float4 t = wg[4 * lane + j];
        h[0] = t.x; h[1] = t.y; h[2] = t.z; h[3] = t.w;
    } else {
        const uint2 t = reinterpret_cast<const uint2 *>(wg)[4 * lane + j];
        h[0] = half_bits_to_float<GT>(t.x & 0xffffu);
        h[1] = half_bits_to_float<GT>(t.x >> 16);
        h[2] = half_bits_to_float<GT>(t.y & 0xffffu);
        h[3] = half_bits_to_float<GT>(t.y >> 16);
    }
    if (LOCO) {
        const float4 t = we[4 * lane + j];
        e[0] = t.x; e[1] = t.y; e[2] = t.z; e[3] = t.w;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = add_rn(h[q], e[q]);     // compensated gradient h
    }
}

// The lane's sixteen codes (element 16l + q of the bucket at code[q]): one 8-byte
// (4-bit) or 16-byte (8-bit) store, bytewise at a ragged end.
template <int BITS>
__device__ __forceinline__ void store_codes(const GArgs &a, int64_t base, int k0, int32_t len,
                                            const uint32_t (&code)[16]) {
    if (BITS == 4) {
        uint2 pk;
        pk.x = code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12) | (code[4] << 16) | (code[5] << 20) |
               (code[6] << 24) | (code[7] << 28);
        pk.y = code[8] | (code[9] << 4) | (code[10] << 8) | (code[11] << 12) | (code[12] << 16) |
               (code[13] << 20) | (code[14] << 24) | (code[15] << 28);
        uint8_t *dst = a.codes + ((base + k0) >> 1);
        if (k0 + 15 < len) {
            *reinterpret_cast<uint2 *>(dst) = pk;
        } else {
            for (int q = 0; 2 * q < len - k0; ++q) dst[q] = (uint8_t)(((q < 4 ? pk.x : pk.y) >> (8 * (q & 3))) & 0xffu);
        }
    } else {
        uint4 pk;
        pk.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        pk.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
        pk.z = code[8] | (code[9] << 8) | (code[10] << 16) | (code[11] << 24);
        pk.w = code[12] | (code[13] << 8) | (code[14] << 16) | (code[15] << 24);
        uint8_t *dst = a.codes + base + k0;
        if (k0 + 15 < len) {
            *reinterpret_cast<uint4 *>(dst) = pk;
        } else {
            for (int q = 0; q < len - k0; ++q) dst[q] = (uint8_t)code[q];
        }
    }
}

// A whole bucket of 1024 staged in LDS (g in wg, LoCo's err in we): pass 1 sums the
// squares of the lane's sixteen values in order (the norm), pass 2 codes them and
// updates the error average group by group, writing it back to the lane's own LDS
// slots; then the error average leaves as contiguous 1 KiB runs and the codes as
// one store per lane.  Every value is formed by the same operations, in the same
// order, as for a bucket held in registers.
template <int BITS, int GT, bool LOCO>
__device__ __forceinline__ void quantize_whole_bucket(const GArgs &a, int64_t b, int64_t base, int lane, float4 *wg,
                                                      float4 *we) {
    const int k0 = 16 * lane;
    float norm;
    double ps = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float h[4], e[4];
        staged_group<GT, LOCO>(wg, we, lane, j, h, e);
#pragma unroll
        for (int q = 0; q < 4; ++q) ps = __fma_rn((double)h[q], (double)h[q], ps);   // each square exact
    }
    if (!norm_from_plain_sum(ps, norm)) {
        DD acc{0.0, 0.0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float h[4], e[4];
            staged_group<GT, LOCO>(wg, we, lane, j, h, e);
#pragma unroll
            for (int q = 0; q < 4; ++q) dd_add_term(acc, (double)h[q] * (double)h[q]);
        }
        norm = norm_of(acc);
    }
    const double rnorm = recip_rn64(norm);
    if (lane == 0) a.norms[b] = norm;
    uint32_t code[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float h[4], e[4];
        staged_group<GT, LOCO>(wg, we, lane, j, h, e);
        const uint64_t blk = (uint64_t)(base + k0 + 4 * j) >> 2;
        const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
        code[4 * j + 0] = qsgd_code<BITS>(h[0], norm, rnorm, r.a);
        code[4 * j + 1] = qsgd_code<BITS>(h[1], norm, rnorm, r.b);
        code[4 * j + 2] = qsgd_code<BITS>(h[2], norm, rnorm, r.c);
        code[4 * j + 3] = qsgd_code<BITS>(h[3], norm, rnorm, r.d);
        if (LOCO) {
            float en[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) en[q] = loco_update<BITS>(a, e[q], h[q], code[4 * j + q], norm);
            we[4 * lane + j] = make_float4(en[0], en[1], en[2], en[3]);
        }
    }
    if (LOCO) {
        __builtin_amdgcn_wave_barrier();
        float4 *dst = reinterpret_cast<float4 *>(a.err + base);
#pragma unroll
        for (int h = 0; h < 4; ++h) st_stream(dst + 64 * h + lane, we[64 * h + lane]);
    }
    store_codes<BITS>(a, base, k0, 1024, code);
    __builtin_amdgcn_wave_barrier();   // the staged bucket is read before the next one overwrites it
}

// Buckets of 1024: one wave per bucket, lane l owns the 16 consecutive elements
// 16l..16l+15; four Philox calls per lane; one 8- or 16-byte store of codes.
// TAIL = false takes the whole buckets: the gradient (and LoCo's error average, both
// ways) moves between HBM and LDS as contiguous 1 KiB runs per wave instruction
// (streaming cache policy) and the lanes read their elements from LDS in both passes
// (quantize_whole_bucket).  TAIL = true takes only the ragged last bucket, its
// elements kept in registers between the norm and the codes; it is a launch of its
// own so that its registers do not set the occupancy of the whole-bucket kernel.
template <int BITS, int GT, bool LOCO, bool TAIL>
__global__ __launch_bounds__(256) void k_qsgd_quantize_1024(GArgs a) {
    __shared__ float4 s_g[4][256];
    __shared__ float4 s_e[4][LOCO ? 256 : 1];
    float4 *const wg = s_g[threadIdx.x >> 6];
    float4 *const we = s_e[threadIdx.x >> 6];
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int64_t n_whole = a.n / 1024;
    for (int64_t b = (TAIL ? n_whole : 0) + wave; b < (TAIL ? a.n_buckets : n_whole); b += nwaves) {
        const int64_t base = b * 1024;
        const int32_t len = (int32_t)min((int64_t)1024, a.n - base);
        const int k0 = 16 * lane;
        float f[16];
        float ea[LOCO ? 16 : 1];
        if (!TAIL) {
            // the bucket goes to LDS only; the lanes read their elements from there in
            // both passes below, so nothing of it stays live in registers
            if (GT == kGradF32) {
                const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + base);
                float4 v[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) v[h] = ld_stream(src + 64 * h + lane);
#pragma unroll
                for (int h = 0; h < 4; ++h) wg[64 * h + lane] = v[h];
            } else {
                const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g) + base);
                uint4 *wu = reinterpret_cast<uint4 *>(wg);
                uint4 v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) v[h] = ld_stream(src + 64 * h + lane);
#pragma unroll
                for (int h = 0; h < 2; ++h) wu[64 * h + lane] = v[h];
            }
            if (LOCO) {
                const float4 *src = reinterpret_cast<const float4 *>(a.err + base);
                float4 v[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) v[h] = ld_stream(src + 64 * h + lane);
#pragma unroll
                for (int h = 0; h < 4; ++h) we[64 * h + lane] = v[h];
            }
            __builtin_amdgcn_wave_barrier();
            quantize_whole_bucket<BITS, GT, LOCO>(a, b, base, lane, wg, we);
            continue;
        } else if (k0 + 15 < len) {
            if (GT == kGradF32) {
                const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + base + k0);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float4 v = src[h];
                    f[4 * h] = v.x; f[4 * h + 1] = v.y; f[4 * h + 2] = v.z; f[4 * h + 3] = v.w;
                }
            } else {
                const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.g) + base + k0);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 v = src[h];
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f[8 * h + 2 * q] = half_bits_to_float<GT>(w[q] & 0xffffu);
                        f[8 * h + 2 * q + 1] = half_bits_to_float<GT>(w[q] >> 16);
                    }
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) f[q] = (k0 + q < len) ? load_grad<GT>(a.g, base + k0 + q) : 0.0f;
        }
        if (LOCO) {
            if (k0 + 15 < len) {
                const float4 *src = reinterpret_cast<const float4 *>(a.err + base + k0);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float4 v = src[h];
                    ea[4 * h] = v.x; ea[4 * h + 1] = v.y; ea[4 * h + 2] = v.z; ea[4 * h + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) ea[q] = (k0 + q < len) ? a.err[base + k0 + q] : 0.0f;
            }
        }
        if (LOCO) {
#pragma unroll
            for (int q = 0; q < 16; ++q) f[q] = add_rn(f[q], ea[q]);     // compensated gradient h
        }
        float norm;
        double ps = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) ps = __fma_rn((double)f[q], (double)f[q], ps);   // each square exact
        if (!norm_from_plain_sum(ps, norm)) {
            DD acc{0.0, 0.0};
#pragma unroll
            for (int q = 0; q < 16; ++q) dd_add_term(acc, (double)f[q] * (double)f[q]);
            norm = norm_of(acc);
        }
        const double rnorm = recip_rn64(norm);
        if (lane == 0) a.norms[b] = norm;
        uint32_t code[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const uint64_t blk = (uint64_t)(base + k0 + 4 * g4) >> 2;
            const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
            code[4 * g4 + 0] = qsgd_code<BITS>(f[4 * g4 + 0], norm, rnorm, r.a);
            code[4 * g4 + 1] = qsgd_code<BITS>(f[4 * g4 + 1], norm, rnorm, r.b);
            code[4 * g4 + 2] = qsgd_code<BITS>(f[4 * g4 + 2], norm, rnorm, r.c);
            code[4 * g4 + 3] = qsgd_code<BITS>(f[4 * g4 + 3], norm, rnorm, r.d);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if (k0 + q >= len) code[q] = 0;
        if (LOCO) {
#pragma unroll
            for (int q = 0; q < 16; ++q) ea[q] = loco_update<BITS>(a, ea[q], f[q], code[q], norm);
            if (k0 + 15 < len) {
                float4 *dst = reinterpret_cast<float4 *>(a.err + base + k0);
#pragma unroll
                for (int h = 0; h < 4; ++h) dst[h] = make_float4(ea[4 * h], ea[4 * h + 1], ea[4 * h + 2], ea[4 * h + 3]);
            } else {
                for (int q = 0; q < len - k0; ++q) a.err[base + k0 + q] = ea[q];
            }
        }
        store_codes<BITS>(a, base, k0, len, code);
    }
}

// The value that is quantized: g, or with LoCo the compensated h = g + err.
template <int GT, bool LOCO>
__device__ __forceinline__ float value_at(const GArgs &a, int64_t i) {
    const float g = load_grad<GT>(a.g, i);
    return LOCO ? add_rn(g, a.err[i]) : g;
}

// Any bucket size (even for 4-bit codes): one wave per bucket, a norm pass and a
// code pass over lane-strided elements (the bucket is in cache for the second);
// each lane writes whole bytes, one Philox call per element.
template <int BITS, int GT, bool LOCO>
__global__ __launch_bounds__(256) void k_qsgd_quantize_generic(GArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t b = wave; b < a.n_buckets; b += nwaves) {
        const int64_t base = b * a.bucket;
        const int32_t len = (int32_t)min((int64_t)a.bucket, a.n - base);
        DD acc{0.0, 0.0};
        for (int k = lane; k < len; k += 64) {
            const double v = (double)value_at<GT, LOCO>(a, base + k);
            dd_add_term(acc, v * v);
        }
        const float norm = norm_of(acc);
        const double rnorm = recip_rn64(norm);
        if (lane == 0) a.norms[b] = norm;
        const int step = BITS == 4 ? 2 : 1;
        for (int k = step * lane; k < len; k += 64 * step) {
            uint32_t byte = 0;
            for (int q = 0; q < step && k + q < len; ++q) {
                const int64_t i = base + k + q;
                const uint64_t blk = (uint64_t)i >> 2;
                const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
                const uint32_t w = (i & 3) == 0 ? r.a : (i & 3) == 1 ? r.b : (i & 3) == 2 ? r.c : r.d;
                const float h = value_at<GT, LOCO>(a, i);
                const uint32_t code = qsgd_code<BITS>(h, norm, rnorm, w);
                if (LOCO) a.err[i] = loco_update<BITS>(a, a.err[i], h, code, norm);
                byte |= code << (4 * q);
            }
            a.codes[BITS == 4 ? ((base + k) >> 1) : (base + k)] = (uint8_t)byte;
        }
    }
}

// ------------------------------------------------ decode and average
struct RArgs {
    const uint8_t *codes;
    int64_t code_stride;
    const float *norms;
    int64_t norm_stride;
    int64_t n;
    int32_t bucket;
    int32_t W;
    float *out_f32;
    uint16_t *out_bf16;
    double sw, rsw;  // s * W and RN64(1 / (s * W))
};

// The 16 codes of one load (8 bytes of 4-bit codes, 16 bytes of 8-bit codes),
// unrolled with compile-time bit positions.
constexpr int kReduceE = 16;
template <int BITS, int K = 0>
struct Accumulate16 {
    static constexpr int PER = 32 / BITS;
    static constexpr int NW = BITS / 2;
    __device__ __forceinline__ static void run(double (&acc)[kReduceE], const uint32_t (&ws)[NW],
                                               const double (&step)[kReduceE]) {
        acc[K] = qsgd_accumulate<BITS, BITS * (K % PER)>(acc[K], ws[K / PER], step[K]);
        Accumulate16<BITS, K + 1>::run(acc, ws, step);
    }
};
template <>
struct Accumulate16<4, 16> {
    __device__ __forceinline__ static void run(double (&)[16], const uint32_t (&)[2], const double (&)[16]) {}
};
template <>
struct Accumulate16<8, 16> {
    __device__ __forceinline__ static void run(double (&)[16], const uint32_t (&)[4], const double (&)[16]) {}
};

// The mean over W: the fp64 sum of the products divided once by s * W, rounded once.
__device__ __forceinline__ float mean_of(const RArgs &a, double acc) { return (float)div_rn64(acc, a.sw, a.rsw); }

__device__ __forceinline__ void store_out(const RArgs &a, int64_t i, float y) {
    if (a.out_f32) a.out_f32[i] = y;
    if (a.out_bf16) a.out_bf16[i] = (uint16_t)float_to_bf16_bits(y);
}

// E = 16 consecutive elements per thread and iteration: one 8-byte (4-bit codes) or
// 16-byte (8-bit) load of every worker's row, 16 fp64 sums live per thread.  With
// the bucket a multiple of E the E elements share one norm per worker.  Sum over workers in fp64, in worker order.  The results of a wave (1024
// consecutive elements) pass through LDS so that every store instruction writes one
// contiguous run (1 KiB of fp32 or bf16), with the streaming cache policy; the waves
// step through the vector together, so every lane takes part in the exchange.
constexpr int kBatch = 4;

template <int BITS, bool SHARED_NORM>
__global__ __launch_bounds__(256) void k_qsgd_reduce(RArgs a) {
    constexpr int E = kReduceE;
    constexpr int NW = BITS / 2;   // 32-bit words per load
    __shared__ float4 s_out[4][64 * E / 4];
    float4 *const sw = s_out[threadIdx.x >> 6];
    const int lane = threadIdx.x & 63;
    const int64_t groups = a.n / E;
    for (int64_t q0 = blockIdx.x * (int64_t)blockDim.x + (threadIdx.x & ~63); q0 < groups;
         q0 += (int64_t)gridDim.x * blockDim.x) {
        const int64_t q = q0 + lane;
        const int64_t i0 = E * q;
        double acc[E];
#pragma unroll
        for (int k = 0; k < E; ++k) acc[k] = 0.0;
        const int64_t b0 = i0 / a.bucket;
        if (q < groups) {
            // workers in batches of kBatch: every load of a batch is issued before its
            // words are decoded, so each thread keeps kBatch 16-byte loads in flight
            for (int w0 = 0; w0 < a.W; w0 += kBatch) {
                uint32_t word[kBatch][NW];
                float nm[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    if (w0 + j < a.W) {
                        const uint8_t *src = a.codes + (int64_t)(w0 + j) * a.code_stride + (int64_t)(E * BITS / 8) * q;
                        if (BITS == 4) {
                            const uint2 v = *reinterpret_cast<const uint2 *>(src);
                            word[j][0] = v.x;
                            word[j][NW > 1 ? 1 : 0] = v.y;
                        } else {
                            const uint4 v = *reinterpret_cast<const uint4 *>(src);
                            word[j][0] = v.x;
                            word[j][NW > 1 ? 1 : 0] = v.y;
                            word[j][NW > 2 ? 2 : 0] = v.z;
                            word[j][NW > 3 ? 3 : 0] = v.w;
                        }
                        nm[j] = SHARED_NORM ? a.norms[(int64_t)(w0 + j) * a.norm_stride + b0] : 0.0f;
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    if (w0 + j >= a.W) break;
                    uint32_t ws[NW];
#pragma unroll
                    for (int h = 0; h < NW; ++h) ws[h] = word[j][h];
                    double sk[E];
                    if (SHARED_NORM) {
                        const double st = (double)nm[j];
#pragma unroll
                        for (int k = 0; k < E; ++k) sk[k] = st;
                    } else {
                        const float *nrow = a.norms + (int64_t)(w0 + j) * a.norm_stride;
#pragma unroll
                        for (int k = 0; k < E; ++k) sk[k] = (double)nrow[(i0 + k) / a.bucket];
                    }
                    Accumulate16<BITS>::run(acc, ws, sk);
                }
            }
        }
        float y[E];
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = mean_of(a, acc[k]);
        // store h of a lane covers the wave's elements 4 (64 h + lane) .. +3 (fp32) or
        // 8 (64 h + lane) .. +7 (bf16), computed by lane 16 h + lane / 4 or 32 h + lane / 2
        if (a.out_f32) {
#pragma unroll
            for (int h = 0; h < E / 4; ++h) sw[4 * lane + h] = make_float4(y[4 * h], y[4 * h + 1], y[4 * h + 2], y[4 * h + 3]);
            __builtin_amdgcn_wave_barrier();
            float4 *o = reinterpret_cast<float4 *>(a.out_f32 + E * q0);
#pragma unroll
            for (int h = 0; h < E / 4; ++h)
                if (q0 + 16 * h + (lane >> 2) < groups) st_stream(o + 64 * h + lane, sw[64 * h + lane]);
            __builtin_amdgcn_wave_barrier();
        }
        if (a.out_bf16) {
            uint4 *su = reinterpret_cast<uint4 *>(sw);
#pragma unroll
            for (int h = 0; h < E / 8; ++h) {
                uint4 pk;
                pk.x = float_to_bf16_bits(y[8 * h + 0]) | (float_to_bf16_bits(y[8 * h + 1]) << 16);
                pk.y = float_to_bf16_bits(y[8 * h + 2]) | (float_to_bf16_bits(y[8 * h + 3]) << 16);
                pk.z = float_to_bf16_bits(y[8 * h + 4]) | (float_to_bf16_bits(y[8 * h + 5]) << 16);
                pk.w = float_to_bf16_bits(y[8 * h + 6]) | (float_to_bf16_bits(y[8 * h + 7]) << 16);
                su[2 * lane + h] = pk;
            }
            __builtin_amdgcn_wave_barrier();
            uint4 *o = reinterpret_cast<uint4 *>(a.out_bf16 + E * q0);
#pragma unroll
            for (int h = 0; h < E / 8; ++h)
                if (q0 + 32 * h + (lane >> 1) < groups) st_stream(o + 64 * h + lane, su[64 * h + lane]);
            __builtin_amdgcn_wave_barrier();
        }
    }
    // ragged tail (n % E elements), one thread each
    const int64_t tail = a.n - E * groups;
    const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (gid < tail) {
        const int64_t i = E * groups + gid;
        double acc = 0.0;
        for (int w = 0; w < a.W; ++w) {
            const uint8_t *row = a.codes + (int64_t)w * a.code_stride;
            const uint32_t c = BITS == 4 ? (uint32_t)(row[i >> 1] >> ((i & 1) * 4)) & 15u : (uint32_t)row[i];
            acc = qsgd_accumulate<BITS, 0>(acc, c, (double)a.norms[(int64_t)w * a.norm_stride + i / a.bucket]);
        }
        store_out(a, i, mean_of(a, acc));
    }
}

static int device_cus() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus;
}

// The launch status of the call's kernels (the first failure, if any).
template <int BITS, int GT, bool LOCO>
static hipError_t launch_quantize(const GArgs &a, unsigned grid, hipStream_t s) {
    if (a.bucket != 1024) {
        hipLaunchKernelGGL((k_qsgd_quantize_generic<BITS, GT, LOCO>), dim3(grid), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    // grid covers the whole buckets; one more workgroup takes a ragged last one
    if (a.n >= 1024) {
        hipLaunchKernelGGL((k_qsgd_quantize_1024<BITS, GT, LOCO, false>), dim3(grid), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.n % 1024) {
        hipLaunchKernelGGL((k_qsgd_quantize_1024<BITS, GT, LOCO, true>), dim3(1), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int BITS, bool LOCO>
static hipError_t launch_quantize_dt(const GArgs &a, onebit_dtype_t dt, unsigned grid, hipStream_t s) {
    if (dt == ONEBIT_BF16) return launch_quantize<BITS, kGradBF16, LOCO>(a, grid, s);
    if (dt == ONEBIT_F16) return launch_quantize<BITS, kGradF16, LOCO>(a, grid, s);
    return launch_quantize<BITS, kGradF32, LOCO>(a, grid, s);
}

// Validation and launch shared by the plain and the LoCo quantizer.
static onebit_status_t quantize_entry(const void *g, onebit_dtype_t g_dtype, float *err, double beta, int64_t n,
                                      int bucket, int bits, uint64_t seed, uint8_t *codes, float *norms,
                                      void *stream) {
    if (n < 0 || bucket < 1 || bucket > 65536 || (bits != 4 && bits != 8)) return ONEBIT_ERR_INVALID;
    if (g_dtype != ONEBIT_F32 && g_dtype != ONEBIT_BF16 && g_dtype != ONEBIT_F16) return ONEBIT_ERR_INVALID;
    if (bits == 4 && (bucket & 1)) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!g || !codes || !norms) return ONEBIT_ERR_INVALID;
    if (!aligned16(g) || !aligned16(codes) || !aligned_to(norms, 4) || (err && !aligned16(err)))
        return ONEBIT_ERR_ALIGN;
    GArgs a{};
    a.g = g;
    a.err = err;
    a.beta = (float)beta;
    a.obeta = (float)(1.0 - beta);
    a.n = n;
    a.n_buckets = (n + bucket - 1) / bucket;
    a.bucket = bucket;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.codes = codes;
    a.norms = norms;
    int64_t blocks = (a.n_buckets + 3) / 4;
    const int64_t cap = (int64_t)device_cus() * 32;
    if (blocks > cap) blocks = cap;
    const unsigned grid = (unsigned)(blocks < 1 ? 1 : blocks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    prof_before(err ? kProfLocoQuantize : kProfQsgdQuantize, s);
    hipError_t e;
    if (bits == 4 && err)
        e = launch_quantize_dt<4, true>(a, g_dtype, grid, s);
    else if (bits == 4)
        e = launch_quantize_dt<4, false>(a, g_dtype, grid, s);
    else if (err)
        e = launch_quantize_dt<8, true>(a, g_dtype, grid, s);
    else
        e = launch_quantize_dt<8, false>(a, g_dtype, grid, s);
    prof_after(s);
    return hip_status(e);
}

template <int BITS>
static void launch_reduce(const RArgs &a, bool shared, unsigned grid, hipStream_t s) {
    if (shared)
        hipLaunchKernelGGL((k_qsgd_reduce<BITS, true>), dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_qsgd_reduce<BITS, false>), dim3(grid), dim3(256), 0, s, a);
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t qsgd_quantize(const void *g, onebit_dtype_t g_dtype, int64_t n, int bucket, int bits,
                                         uint64_t seed, uint8_t *codes, float *norms, void *stream) {
    return quantize_entry(g, g_dtype, nullptr, 0.0, n, bucket, bits, seed, codes, norms, stream);
}

extern "C" onebit_status_t loco_quantize(const void *g, onebit_dtype_t g_dtype, float *err_avg, int64_t n, int bucket,
                                         int bits, double beta, uint64_t seed, uint8_t *codes, float *norms,
                                         void *stream) {
    if (n > 0 && !err_avg) return ONEBIT_ERR_INVALID;
    if (!(beta >= 0.0 && beta <= 1.0)) return ONEBIT_ERR_INVALID;
    return quantize_entry(g, g_dtype, err_avg, beta, n, bucket, bits, seed, codes, norms, stream);
}

extern "C" onebit_status_t qsgd_reduce(int W, const uint8_t *codes, int64_t code_stride, const float *norms,
                                       int64_t norm_stride, int64_t n, int bucket, int bits, float *out_f32,
                                       uint16_t *out_bf16, void *stream) {
    if (W < 1 || W > 65536 || n < 0 || bucket < 1 || bucket > 65536 || (bits != 4 && bits != 8))
        return ONEBIT_ERR_INVALID;
    if (bits == 4 && (bucket & 1)) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    const int64_t code_bytes = bits == 4 ? (n + 1) / 2 : n;
    const int64_t n_buckets = (n + bucket - 1) / bucket;
    if (!codes || !norms || (!out_f32 && !out_bf16)) return ONEBIT_ERR_INVALID;
    if (W > 1 && (code_stride < code_bytes || norm_stride < n_buckets)) return ONEBIT_ERR_INVALID;
    if (!aligned16(codes) || (W > 1 && code_stride % 16 != 0) || !aligned_to(norms, 4)) return ONEBIT_ERR_ALIGN;
    if ((out_f32 && !aligned16(out_f32)) || (out_bf16 && !aligned16(out_bf16))) return ONEBIT_ERR_ALIGN;
    RArgs a{};
    a.codes = codes;
    a.code_stride = code_stride;
    a.norms = norms;
    a.norm_stride = norm_stride;
    a.n = n;
    a.bucket = bucket;
    a.W = W;
    a.out_f32 = out_f32;
    a.out_bf16 = out_bf16;
    int64_t blocks = (n / kReduceE + 255) / 256;
    const int64_t cap = (int64_t)device_cus() * 16;
    if (blocks > cap) blocks = cap;
    const unsigned grid = (unsigned)(blocks < 1 ? 1 : blocks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    a.sw = (double)((1u << (bits - 1)) - 1u) * (double)W;
    a.rsw = 1.0 / a.sw;
    const bool shared = bucket % kReduceE == 0;
    prof_before(kProfQsgdReduce, s);
    if (bits == 4)
        launch_reduce<4>(a, shared, grid, s);
    else
        launch_reduce<8>(a, shared, grid, s);
    prof_after(s);
    return hip_status(hipGetLastError());
}

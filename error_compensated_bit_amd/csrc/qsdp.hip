// qsdp.hip -- QSDP-style unbiased stochastic rounding of bf16 weights and its
// inverse (QSDP review, "proposed method": each weight goes to one of its two
// nearest quantization levels at random, with expectation equal to the weight).
// Levels: 2^bits evenly spaced over each bucket's [min, max].  Random words:
// Philox4x32-10 (Salmon et al., SC'11) keyed by the seed, counter = element
// index / 4, word = element index % 4, so one Philox call serves four
// consecutive elements.
//
// One wave64 per bucket: lane l handles element groups 4(l + 64k); the bucket's
// min and max come from a wave-wide reduction on order-preserving integer keys
// (so -0 < +0 and the result does not depend on reduction order).
#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "quant_common.h"

namespace onebit {

// float -> int32 key whose signed order is the IEEE total order on non-NaN values
__device__ __forceinline__ int32_t order_key(float f) {
    const int32_t s = __float_as_int(f);
    return s >= 0 ? s : (s ^ 0x7fffffff);
}
__device__ __forceinline__ float key_to_float(int32_t k) { return __int_as_float(k >= 0 ? k : (k ^ 0x7fffffff)); }

// The same order on bf16 values, two at a time in the halves of a 32-bit word
// (packed 16-bit integer operations), and the 32-bit key of a 16-bit one:
// order_key(float(bf16 b)) is key16(b) << 16, with the low half all ones when the
// value is negative.
typedef short short2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ short2_v bf16x2_keys(uint32_t w) {
    const short2_v v = __builtin_bit_cast(short2_v, w);
    return v ^ ((v >> (short)15) & (short2_v)(short)0x7fff);
}
__device__ __forceinline__ int32_t key16_to_key32(int32_t k) {
    return (int32_t)((uint32_t)k << 16) | (k < 0 ? 0xffff : 0);
}

__device__ __forceinline__ int32_t wave_min_i(int32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int32_t wave_max_i(int32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
    return v;
}

struct QArgs {
    const uint16_t *x;
    int64_t n;
    int64_t n_buckets;
    int32_t bucket;
    int32_t bits;
    uint32_t k0, k1;  // Philox key (seed low / high word)
    uint8_t *codes;
    float *bmin, *bmax;
    // dequantize
    const uint8_t *in_codes;
    const float *in_min, *in_max;
    uint16_t *out_bf16;
    float *out_f32;
};

// Stochastic rounding of one element given its uniform word; rdelta = RN64(1 / delta).
template <int BITS>
__device__ __forceinline__ uint32_t sr_code(float x, float mn, float delta, double rdelta, uint32_t u) {
    constexpr float L = (float)((1 << BITS) - 1);
    if (delta == 0.0f) return 0u;
    const float t = div_by_recip(sub_rn(x, mn), rdelta);  // = fl32((x - mn) / delta)
    const float k = fminf(floorf(t), L);
    const float p = sub_rn(t, k);                          // exact
    // floor(p * 2^32), exact; p >= 1 only when k was clamped to L, where any
    // threshold gives code L after the final clamp
    const uint32_t thr = p < 1.0f ? (uint32_t)ldexpf(p, 32) : 0xffffffffu;
    const uint32_t code = (uint32_t)k + (u < thr ? 1u : 0u);
    return code > (uint32_t)L ? (uint32_t)L : code;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_qsdp_quantize(QArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    constexpr float L = (float)((1 << BITS) - 1);
    for (int64_t b = wave; b < a.n_buckets; b += nwaves) {
        const int64_t base = b * a.bucket;
        const int32_t len = (int32_t)min((int64_t)a.bucket, a.n - base);
        // pass over the bucket: min / max keys
        int32_t kmin = 0x7fffffff, kmax = (int32_t)0x80000000;
        for (int g4 = 4 * lane; g4 < len; g4 += 256) {
            const int64_t i = base + g4;
            if (g4 + 3 < len) {
                const uint2 h = *reinterpret_cast<const uint2 *>(a.x + i);
                const float f0 = bf16_bits_to_float(h.x & 0xffffu), f1 = bf16_bits_to_float(h.x >> 16);
                const float f2 = bf16_bits_to_float(h.y & 0xffffu), f3 = bf16_bits_to_float(h.y >> 16);
                kmin = min(kmin, min(min(order_key(f0), order_key(f1)), min(order_key(f2), order_key(f3))));
                kmax = max(kmax, max(max(order_key(f0), order_key(f1)), max(order_key(f2), order_key(f3))));
            } else {
                for (int q = 0; q < 4 && g4 + q < len; ++q) {
                    const int32_t k = order_key(bf16_bits_to_float(a.x[i + q]));
                    kmin = min(kmin, k);
                    kmax = max(kmax, k);
                }
            }
        }
        kmin = wave_min_i(kmin);
        kmax = wave_max_i(kmax);
        const float mn = key_to_float(kmin), mx = key_to_float(kmax);
        const float delta = __fdiv_rn(sub_rn(mx, mn), L);
        const double rdelta = recip_rn64(delta);
        if (lane == 0) {
            a.bmin[b] = mn;
            a.bmax[b] = mx;
        }
        // second pass (the bucket is in L2 / L1): codes
        for (int g4 = 4 * lane; g4 < len; g4 += 256) {
            const int64_t i = base + g4;
            float f[4];
            if (g4 + 3 < len) {
                const uint2 h = *reinterpret_cast<const uint2 *>(a.x + i);
                f[0] = bf16_bits_to_float(h.x & 0xffffu);
                f[1] = bf16_bits_to_float(h.x >> 16);
                f[2] = bf16_bits_to_float(h.y & 0xffffu);
                f[3] = bf16_bits_to_float(h.y >> 16);
            } else {
                for (int q = 0; q < 4; ++q) f[q] = (g4 + q < len) ? bf16_bits_to_float(a.x[i + q]) : mn;
            }
            const uint64_t blk = (uint64_t)i >> 2;
            const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
            uint32_t c0 = sr_code<BITS>(f[0], mn, delta, rdelta, r.a);
            uint32_t c1 = sr_code<BITS>(f[1], mn, delta, rdelta, r.b);
            uint32_t c2 = sr_code<BITS>(f[2], mn, delta, rdelta, r.c);
            uint32_t c3 = sr_code<BITS>(f[3], mn, delta, rdelta, r.d);
            if (g4 + 1 >= len) c1 = 0;
            if (g4 + 2 >= len) c2 = 0;
            if (g4 + 3 >= len) c3 = 0;
            if (BITS == 4) {
                if (g4 + 3 < len) {
                    *reinterpret_cast<uint16_t *>(a.codes + (i >> 1)) =
                        (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
                } else {
                    a.codes[i >> 1] = (uint8_t)(c0 | (c1 << 4));
                    if (g4 + 2 < len) a.codes[(i >> 1) + 1] = (uint8_t)(c2 | (c3 << 4));
                }
            } else {
                if (g4 + 3 < len) {
                    *reinterpret_cast<uint32_t *>(a.codes + i) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
                } else {
                    a.codes[i] = (uint8_t)c0;
                    if (g4 + 1 < len) a.codes[i + 1] = (uint8_t)c1;
                    if (g4 + 2 < len) a.codes[i + 2] = (uint8_t)c2;
                }
            }
        }
    }
}

// Buckets of exactly 1024 elements (the common configuration): one wave per
// bucket, lane l owns the 16 consecutive elements 16l..16l+15, loaded as two
// 16-byte vectors and kept in registers across the min/max and code passes;
// four Philox calls per lane; codes leave as one 8- or 16-byte store.
__device__ __forceinline__ void unpack8(uint4 h, float (&f)[8]) {
    f[0] = bf16_bits_to_float(h.x & 0xffffu); f[1] = bf16_bits_to_float(h.x >> 16);
    f[2] = bf16_bits_to_float(h.y & 0xffffu); f[3] = bf16_bits_to_float(h.y >> 16);
    f[4] = bf16_bits_to_float(h.z & 0xffffu); f[5] = bf16_bits_to_float(h.z >> 16);
    f[6] = bf16_bits_to_float(h.w & 0xffffu); f[7] = bf16_bits_to_float(h.w >> 16);
}

template <int BITS>
// six waves per SIMD (at most 80 VGPRs): the 4-bit variant otherwise takes 82 and runs five
__global__ __launch_bounds__(256, 6) void k_qsdp_quantize_1024(QArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    constexpr float L = (float)((1 << BITS) - 1);
    const int64_t n_full = a.n >> 10;                 // buckets with all 1024 elements
    const int k0 = 16 * lane;
    // the next full bucket's 32 bytes per lane are loaded while this one is coded
    uint4 nx0 = make_uint4(0u, 0u, 0u, 0u), nx1 = nx0;
    if (wave < n_full) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.x + wave * 1024 + k0);
        nx0 = src[0];
        nx1 = src[1];
    }
    for (int64_t b = wave; b < a.n_buckets; b += nwaves) {
        const int64_t base = b * 1024;
        const int32_t len = (int32_t)min((int64_t)1024, a.n - base);
        const uint4 h0 = nx0, h1 = nx1;
        if (b + nwaves < n_full) {
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (b + nwaves) * 1024 + k0);
            nx0 = src[0];
            nx1 = src[1];
        }
        float f[16];
        int32_t kmin = 0x7fffffff, kmax = (int32_t)0x80000000;
        if (b < n_full) {
            const uint32_t w[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            short2_v kmn = bf16x2_keys(w[0]), kmx = kmn;
#pragma unroll
            for (int q = 1; q < 8; ++q) {
                const short2_v k = bf16x2_keys(w[q]);
                kmn = __builtin_elementwise_min(kmn, k);
                kmx = __builtin_elementwise_max(kmx, k);
            }
            kmin = key16_to_key32(min((int32_t)kmn.x, (int32_t)kmn.y));
            kmax = key16_to_key32(max((int32_t)kmx.x, (int32_t)kmx.y));
            float lo[8], hi[8];
            unpack8(h0, lo);
            unpack8(h1, hi);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                f[q] = lo[q];
                f[8 + q] = hi[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                f[q] = (k0 + q < len) ? bf16_bits_to_float(a.x[base + k0 + q]) : 0.0f;
                if (k0 + q < len) {
                    kmin = min(kmin, order_key(f[q]));
                    kmax = max(kmax, order_key(f[q]));
                }
            }
        }
        kmin = wave_min_i(kmin);
        kmax = wave_max_i(kmax);
        const float mn = key_to_float(kmin), mx = key_to_float(kmax);
        const float delta = __fdiv_rn(sub_rn(mx, mn), L);
        const double rdelta = recip_rn64(delta);
        if (lane == 0) {
            a.bmin[b] = mn;
            a.bmax[b] = mx;
        }
        uint32_t code[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint64_t blk = (uint64_t)(base + k0 + 4 * g) >> 2;
            const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
            code[4 * g + 0] = sr_code<BITS>(f[4 * g + 0], mn, delta, rdelta, r.a);
            code[4 * g + 1] = sr_code<BITS>(f[4 * g + 1], mn, delta, rdelta, r.b);
            code[4 * g + 2] = sr_code<BITS>(f[4 * g + 2], mn, delta, rdelta, r.c);
            code[4 * g + 3] = sr_code<BITS>(f[4 * g + 3], mn, delta, rdelta, r.d);
        }
        if (b >= n_full) {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (k0 + q >= len) code[q] = 0;
        }
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
}

// Buckets of 1024, kDeqBatch buckets per wave and iteration: the codes and bucket
// bounds of all of them are loaded before any is decoded, so each wave keeps
// several loads in flight while it writes (the stores outweigh the loads 4:1 or
// 2:1 and need no wait).  A lane takes eight consecutive elements at 8*lane and
// at 512 + 8*lane of the bucket, so every store instruction of a wave writes one
// contiguous 1 KiB run of bf16 outputs (whole cache lines), with the streaming
// cache policy.
constexpr int kDeqBatch = 4;
constexpr int kDeqWords = 2;  // code words per lane and half-bucket (4-bit uses one)

// The fp32 output of a whole half-bucket passes through the wave's LDS buffer `wl`
// (128 16-byte slots), so that its stores are contiguous 1 KiB runs too.
template <int BITS>
__device__ __forceinline__ void dequant8_store(const QArgs &a, int64_t base, int32_t len, int k0, float mn,
                                              float delta, const uint32_t (&wv)[kDeqWords], float4 *wl,
                                              bool half_whole, int64_t half_base) {
    uint32_t code[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        code[q] = BITS == 4 ? (wv[0] >> (4 * q)) & 15u : (wv[q >> 2] >> (8 * (q & 3))) & 255u;
    float y[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) y[q] = add_rn(mn, mul_rn((float)code[q], delta));
    const int64_t i0 = base + k0;
    if (a.out_f32 && half_whole) {
        const int lane = threadIdx.x & 63;
        wl[2 * lane] = make_float4(y[0], y[1], y[2], y[3]);
        wl[2 * lane + 1] = make_float4(y[4], y[5], y[6], y[7]);
        __builtin_amdgcn_wave_barrier();
        float4 *o = reinterpret_cast<float4 *>(a.out_f32 + half_base);
        st_stream(o + lane, wl[lane]);
        st_stream(o + 64 + lane, wl[64 + lane]);
        __builtin_amdgcn_wave_barrier();
    }
    if (k0 + 7 < len) {
        if (a.out_f32 && !half_whole) {
            float4 *o = reinterpret_cast<float4 *>(a.out_f32 + i0);
            o[0] = make_float4(y[0], y[1], y[2], y[3]);
            o[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
        if (a.out_bf16) {
            uint4 pk;
            pk.x = float_to_bf16_bits(y[0]) | (float_to_bf16_bits(y[1]) << 16);
            pk.y = float_to_bf16_bits(y[2]) | (float_to_bf16_bits(y[3]) << 16);
            pk.z = float_to_bf16_bits(y[4]) | (float_to_bf16_bits(y[5]) << 16);
            pk.w = float_to_bf16_bits(y[6]) | (float_to_bf16_bits(y[7]) << 16);
            st_stream(reinterpret_cast<uint4 *>(a.out_bf16 + i0), pk);
        }
    } else {
        for (int q = 0; q < len - k0; ++q) {
            if (a.out_f32) a.out_f32[i0 + q] = y[q];
            if (a.out_bf16) a.out_bf16[i0 + q] = (uint16_t)float_to_bf16_bits(y[q]);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_qsdp_dequantize_1024(QArgs a) {
    __shared__ float4 s_y[4][128];
    float4 *const wl = s_y[threadIdx.x >> 6];
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    constexpr float L = (float)((1 << BITS) - 1);
    for (int64_t b0 = wave * kDeqBatch; b0 < a.n_buckets; b0 += nwaves * kDeqBatch) {
        uint32_t wv[kDeqBatch][2][kDeqWords];
        float mn[kDeqBatch], mx[kDeqBatch];
#pragma unroll
        for (int u = 0; u < kDeqBatch; ++u) {
            const int64_t b = b0 + u;
#pragma unroll
            for (int h = 0; h < 2; ++h) wv[u][h][0] = wv[u][h][1] = 0u;
            mn[u] = mx[u] = 0.0f;
            if (b < a.n_buckets) {
                const int64_t base = b * 1024;
                const int32_t len = (int32_t)min((int64_t)1024, a.n - base);
                mn[u] = a.in_min[b];
                mx[u] = a.in_max[b];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k0 = 8 * lane + 512 * h;
                    if (k0 + 7 < len) {
                        if (BITS == 4) {
                            wv[u][h][0] = *reinterpret_cast<const uint32_t *>(a.in_codes + ((base + k0) >> 1));
                        } else {
                            const uint2 w = *reinterpret_cast<const uint2 *>(a.in_codes + base + k0);
                            wv[u][h][0] = w.x;
                            wv[u][h][1] = w.y;
                        }
                    } else if (k0 < len) {
                        if (BITS == 4) {
                            const uint8_t *src = a.in_codes + ((base + k0) >> 1);
                            for (int q = 0; 2 * q < len - k0; ++q) wv[u][h][0] |= (uint32_t)src[q] << (8 * q);
                        } else {
                            const uint8_t *src = a.in_codes + base + k0;
                            for (int q = 0; q < len - k0; ++q) wv[u][h][q >> 2] |= (uint32_t)src[q] << (8 * (q & 3));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kDeqBatch; ++u) {
            const int64_t b = b0 + u;
            if (b >= a.n_buckets) break;
            const int64_t base = b * 1024;
            const int32_t len = (int32_t)min((int64_t)1024, a.n - base);
            const float delta = __fdiv_rn(sub_rn(mx[u], mn[u]), L);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k0 = 8 * lane + 512 * h;
                if (k0 < len)
                    dequant8_store<BITS>(a, base, len, k0, mn[u], delta, wv[u][h], wl, len >= 512 * (h + 1),
                                         base + 512 * h);
            }
        }
    }
}

// Generic bucket size (not a multiple of 4): one Philox call per element.
template <int BITS>
__global__ __launch_bounds__(256) void k_qsdp_quantize_generic(QArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    constexpr float L = (float)((1 << BITS) - 1);
    for (int64_t b = wave; b < a.n_buckets; b += nwaves) {
        const int64_t base = b * a.bucket;
        const int32_t len = (int32_t)min((int64_t)a.bucket, a.n - base);
        int32_t kmin = 0x7fffffff, kmax = (int32_t)0x80000000;
        for (int k = lane; k < len; k += 64) {
            const int32_t key = order_key(bf16_bits_to_float(a.x[base + k]));
            kmin = min(kmin, key);
            kmax = max(kmax, key);
        }
        kmin = wave_min_i(kmin);
        kmax = wave_max_i(kmax);
        const float mn = key_to_float(kmin), mx = key_to_float(kmax);
        const float delta = __fdiv_rn(sub_rn(mx, mn), L);
        const double rdelta = recip_rn64(delta);
        if (lane == 0) {
            a.bmin[b] = mn;
            a.bmax[b] = mx;
        }
        // 8-bit: one byte per element; 4-bit: bucket is even, each lane owns whole bytes
        const int step = BITS == 4 ? 2 : 1;
        for (int k = step * lane; k < len; k += 64 * step) {
            uint32_t byte = 0;
            for (int q = 0; q < step && k + q < len; ++q) {
                const int64_t i = base + k + q;
                const uint64_t blk = (uint64_t)i >> 2;
                const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, a.k0, a.k1);
                const uint32_t w = (i & 3) == 0 ? r.a : (i & 3) == 1 ? r.b : (i & 3) == 2 ? r.c : r.d;
                byte |= sr_code<BITS>(bf16_bits_to_float(a.x[i]), mn, delta, rdelta, w) << (4 * q);
            }
            a.codes[BITS == 4 ? ((base + k) >> 1) : (base + k)] = (uint8_t)byte;
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_qsdp_dequantize(QArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    constexpr float L = (float)((1 << BITS) - 1);
    for (int64_t b = wave; b < a.n_buckets; b += nwaves) {
        const int64_t base = b * a.bucket;
        const int32_t len = (int32_t)min((int64_t)a.bucket, a.n - base);
        const float mn = a.in_min[b];
        const float delta = __fdiv_rn(sub_rn(a.in_max[b], mn), L);
        const bool fast = (a.bucket & 3) == 0;
        for (int g4 = 4 * lane; g4 < len; g4 += 256) {
            const int64_t i = base + g4;
            uint32_t c[4];
            if (fast && g4 + 3 < len) {
                if (BITS == 4) {
                    const uint32_t w = *reinterpret_cast<const uint16_t *>(a.in_codes + (i >> 1));
                    c[0] = w & 15u; c[1] = (w >> 4) & 15u; c[2] = (w >> 8) & 15u; c[3] = (w >> 12) & 15u;
                } else {
                    const uint32_t w = *reinterpret_cast<const uint32_t *>(a.in_codes + i);
                    c[0] = w & 255u; c[1] = (w >> 8) & 255u; c[2] = (w >> 16) & 255u; c[3] = w >> 24;
                }
            } else {
                for (int q = 0; q < 4; ++q) {
                    const int64_t j = i + q;
                    c[q] = (g4 + q < len) ? (BITS == 4 ? (a.in_codes[j >> 1] >> ((j & 1) * 4)) & 15u : a.in_codes[j]) : 0u;
                }
            }
            float y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) y[q] = add_rn(mn, mul_rn((float)c[q], delta));
            if (fast && g4 + 3 < len) {
                if (a.out_f32) *reinterpret_cast<float4 *>(a.out_f32 + i) = make_float4(y[0], y[1], y[2], y[3]);
                if (a.out_bf16) {
                    uint2 pk;
                    pk.x = float_to_bf16_bits(y[0]) | (float_to_bf16_bits(y[1]) << 16);
                    pk.y = float_to_bf16_bits(y[2]) | (float_to_bf16_bits(y[3]) << 16);
                    *reinterpret_cast<uint2 *>(a.out_bf16 + i) = pk;
                }
            } else {
                for (int q = 0; q < 4 && g4 + q < len; ++q) {
                    if (a.out_f32) a.out_f32[i + q] = y[q];
                    if (a.out_bf16) a.out_bf16[i + q] = (uint16_t)float_to_bf16_bits(y[q]);
                }
            }
        }
    }
}

// ------------------------------------------------------ error statistics
// Fixed grid and fixed reduction tree: the sums are bitwise reproducible.
constexpr int kStatBlocks = 1024;

__device__ __forceinline__ double block_sum_d(double v, double *s_red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    __syncthreads();
    return t;
}

// partials[2b] = sum (y - x), partials[2b+1] = sum (y - x)^2 over block b's share;
// ysum += y when given.
// Two consecutive elements per thread and access, so that every access
// instruction of a wave covers whole contiguous lines (256 B of weights, 512 B of
// y, 1 KiB of ysum), with kStatU pairs per thread in flight; fp64 running sums in a
// fixed order (bitwise reproducible).  An odd last element is taken by thread 0.
constexpr int kStatU = 4;

__device__ __forceinline__ void ld_f64x2(const double *p, double &a, double &b) {
    const uint4 w = ld_stream(reinterpret_cast<const uint4 *>(p));
    a = __hiloint2double((int)w.y, (int)w.x);
    b = __hiloint2double((int)w.w, (int)w.z);
}
__device__ __forceinline__ void st_f64x2(double *p, double a, double b) {
    const uint64_t ua = (uint64_t)__double_as_longlong(a), ub = (uint64_t)__double_as_longlong(b);
    st_stream(reinterpret_cast<uint4 *>(p), make_uint4((uint32_t)ua, (uint32_t)(ua >> 32), (uint32_t)ub, (uint32_t)(ub >> 32)));
}

__device__ __forceinline__ void stat_add(double &s1, double &s2, float yv, uint32_t xbits) {
    const double d = (double)yv - (double)bf16_bits_to_float(xbits);
    s1 += d;
    s2 += d * d;
}

__global__ __launch_bounds__(256) void k_qsdp_stats(const uint16_t *x, const float *y, int64_t n, double *ysum,
                                                     double *partials) {
    __shared__ double s_red[4];
    double s1 = 0.0, s2 = 0.0;
    const int64_t pairs = n / 2;
    const int64_t span = (int64_t)blockDim.x * kStatU;
    for (int64_t base = blockIdx.x * span; base < pairs; base += (int64_t)gridDim.x * span) {
        uint32_t xx[kStatU];
        uint2 yy[kStatU];
        double ya[kStatU], yb[kStatU];
#pragma unroll
        for (int u = 0; u < kStatU; ++u) {
            const int64_t p = base + u * (int64_t)blockDim.x + threadIdx.x;
            if (p < pairs) {
                xx[u] = ld_stream(reinterpret_cast<const uint32_t *>(x + 2 * p));
                yy[u] = ld_stream(reinterpret_cast<const uint2 *>(y + 2 * p));
                if (ysum) ld_f64x2(ysum + 2 * p, ya[u], yb[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kStatU; ++u) {
            const int64_t p = base + u * (int64_t)blockDim.x + threadIdx.x;
            if (p < pairs) {
                const float y0 = __uint_as_float(yy[u].x), y1 = __uint_as_float(yy[u].y);
                stat_add(s1, s2, y0, xx[u] & 0xffffu);
                stat_add(s1, s2, y1, xx[u] >> 16);
                if (ysum) st_f64x2(ysum + 2 * p, ya[u] + (double)y0, yb[u] + (double)y1);
            }
        }
    }
    if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0) {
        const int64_t i = n - 1;
        stat_add(s1, s2, y[i], x[i]);
        if (ysum) ysum[i] += (double)y[i];
    }
    const double t1 = block_sum_d(s1, s_red);
    const double t2 = block_sum_d(s2, s_red);
    if (threadIdx.x == 0) {
        partials[2 * blockIdx.x] = t1;
        partials[2 * blockIdx.x + 1] = t2;
    }
}

// partials[b] = sum |ysum / seeds - x| over block b's share (same access pattern)
__global__ __launch_bounds__(256) void k_qsdp_mae(const uint16_t *x, const double *ysum, int64_t n, double inv_seeds,
                                                   double *partials) {
    __shared__ double s_red[4];
    double s = 0.0;
    const int64_t pairs = n / 2;
    const int64_t span = (int64_t)blockDim.x * kStatU;
    for (int64_t base = blockIdx.x * span; base < pairs; base += (int64_t)gridDim.x * span) {
        uint32_t xx[kStatU];
        double ya[kStatU], yb[kStatU];
#pragma unroll
        for (int u = 0; u < kStatU; ++u) {
            const int64_t p = base + u * (int64_t)blockDim.x + threadIdx.x;
            if (p < pairs) {
                xx[u] = ld_stream(reinterpret_cast<const uint32_t *>(x + 2 * p));
                ld_f64x2(ysum + 2 * p, ya[u], yb[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kStatU; ++u) {
            const int64_t p = base + u * (int64_t)blockDim.x + threadIdx.x;
            if (p < pairs) {
                s += fabs(ya[u] * inv_seeds - (double)bf16_bits_to_float(xx[u] & 0xffffu));
                s += fabs(yb[u] * inv_seeds - (double)bf16_bits_to_float(xx[u] >> 16));
            }
        }
    }
    if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0)
        s += fabs(ysum[n - 1] * inv_seeds - (double)bf16_bits_to_float(x[n - 1]));
    const double t = block_sum_d(s, s_red);
    if (threadIdx.x == 0) partials[blockIdx.x] = t;
}

// out[k] += sum_b partials[b * width + k], k < width, in block order
__global__ __launch_bounds__(256) void k_reduce_partials(const double *partials, int width, double *out, int add) {
    __shared__ double s_red[4];
    for (int k = 0; k < width; ++k) {
        double v = 0.0;
        for (int b = threadIdx.x; b < kStatBlocks; b += 256) v += partials[b * width + k];
        const double t = block_sum_d(v, s_red);
        if (threadIdx.x == 0) out[k] = add ? out[k] + t : t;
    }
}

static unsigned grid_for(int64_t n_buckets) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int64_t blocks = (n_buckets + 3) / 4;
    const int64_t cap = (int64_t)cus * 32;
    if (blocks > cap) blocks = cap;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t qsdp_quantize(const uint16_t *x_bf16, int64_t n, int bucket, int bits, uint64_t seed,
                                         uint8_t *codes, float *bucket_min, float *bucket_max, void *stream) {
    if (n < 0 || bucket < 1 || bucket > 65536 || (bits != 4 && bits != 8)) return ONEBIT_ERR_INVALID;
    if (bits == 4 && (bucket & 1)) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!x_bf16 || !codes || !bucket_min || !bucket_max) return ONEBIT_ERR_INVALID;
    if (!aligned16(x_bf16) || !aligned16(codes) || !aligned_to(bucket_min, 4) || !aligned_to(bucket_max, 4))
        return ONEBIT_ERR_ALIGN;
    QArgs a{};
    a.x = x_bf16;
    a.n = n;
    a.n_buckets = (n + bucket - 1) / bucket;
    a.bucket = bucket;
    a.bits = bits;
    a.k0 = (uint32_t)seed;
    a.k1 = (uint32_t)(seed >> 32);
    a.codes = codes;
    a.bmin = bucket_min;
    a.bmax = bucket_max;
    const unsigned grid = grid_for(a.n_buckets);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool fast = (bucket & 3) == 0;
    prof_before(kProfQuantize, s);
    if (bucket == 1024 && bits == 4)
        hipLaunchKernelGGL(k_qsdp_quantize_1024<4>, dim3(grid), dim3(256), 0, s, a);
    else if (bucket == 1024)
        hipLaunchKernelGGL(k_qsdp_quantize_1024<8>, dim3(grid), dim3(256), 0, s, a);
    else if (bits == 4 && fast)
        hipLaunchKernelGGL(k_qsdp_quantize<4>, dim3(grid), dim3(256), 0, s, a);
    else if (bits == 4)
        hipLaunchKernelGGL(k_qsdp_quantize_generic<4>, dim3(grid), dim3(256), 0, s, a);
    else if (fast)
        hipLaunchKernelGGL(k_qsdp_quantize<8>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_qsdp_quantize_generic<8>, dim3(grid), dim3(256), 0, s, a);
    prof_after(s);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t qsdp_dequantize(const uint8_t *codes, const float *bucket_min, const float *bucket_max,
                                           int64_t n, int bucket, int bits, uint16_t *out_bf16, float *out_f32,
                                           void *stream) {
    if (n < 0 || bucket < 1 || bucket > 65536 || (bits != 4 && bits != 8)) return ONEBIT_ERR_INVALID;
    if (bits == 4 && (bucket & 1)) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!codes || !bucket_min || !bucket_max) return ONEBIT_ERR_INVALID;
    if (!aligned16(codes) || !aligned_to(bucket_min, 4) || !aligned_to(bucket_max, 4)) return ONEBIT_ERR_ALIGN;
    if ((out_bf16 && !aligned16(out_bf16)) || (out_f32 && !aligned16(out_f32))) return ONEBIT_ERR_ALIGN;
    QArgs a{};
    a.n = n;
    a.n_buckets = (n + bucket - 1) / bucket;
    a.bucket = bucket;
    a.bits = bits;
    a.in_codes = codes;
    a.in_min = bucket_min;
    a.in_max = bucket_max;
    a.out_bf16 = out_bf16;
    a.out_f32 = out_f32;
    const unsigned grid = grid_for(a.n_buckets);
    hipStream_t s = static_cast<hipStream_t>(stream);
    prof_before(kProfDequantize, s);
    if (bucket == 1024 && bits == 4)
        hipLaunchKernelGGL(k_qsdp_dequantize_1024<4>, dim3(grid), dim3(256), 0, s, a);
    else if (bucket == 1024)
        hipLaunchKernelGGL(k_qsdp_dequantize_1024<8>, dim3(grid), dim3(256), 0, s, a);
    else if (bits == 4)
        hipLaunchKernelGGL(k_qsdp_dequantize<4>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_qsdp_dequantize<8>, dim3(grid), dim3(256), 0, s, a);
    prof_after(s);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t qsdp_error_stats(const uint16_t *x_bf16, const float *y, int64_t n, double *ysum,
                                            double *sums, double *partials, void *stream) {
    if (n < 0 || !sums || !partials) return ONEBIT_ERR_INVALID;
    if (n > 0 && (!x_bf16 || !y)) return ONEBIT_ERR_INVALID;
    if (!aligned_to(sums, 8) || !aligned_to(partials, 8) || (ysum && !aligned16(ysum))) return ONEBIT_ERR_ALIGN;
    if (n > 0 && (!aligned16(x_bf16) || !aligned16(y))) return ONEBIT_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    prof_before(kProfFinalize, s);
    hipLaunchKernelGGL(k_qsdp_stats, dim3(kStatBlocks), dim3(256), 0, s, x_bf16, y, n, ysum, partials);
    hipLaunchKernelGGL(k_reduce_partials, dim3(1), dim3(256), 0, s, (const double *)partials, 2, sums, 1);
    prof_after(s);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t qsdp_mean_abs_error(const uint16_t *x_bf16, const double *ysum, int64_t n, int seeds,
                                               double *out, double *partials, void *stream) {
    if (n < 1 || seeds < 1 || !x_bf16 || !ysum || !out || !partials) return ONEBIT_ERR_INVALID;
    if (!aligned16(ysum) || !aligned16(x_bf16) || !aligned_to(out, 8) || !aligned_to(partials, 8)) return ONEBIT_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_qsdp_mae, dim3(kStatBlocks), dim3(256), 0, s, x_bf16, ysum, n, 1.0 / (double)seeds, partials);
    hipLaunchKernelGGL(k_reduce_partials, dim3(1), dim3(256), 0, s, (const double *)partials, 1, out, 0);
    return hip_status(hipGetLastError());
}

// device_common.h -- gfx950 device helpers shared by the library's kernels:
// exact binary32 arithmetic, bf16 conversion, double-double sums, wave64 lane
// exchange, single-location agent-scope atomics, Philox4x32-10.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace onebit {

// ------------------------------------------------------------- geometry
constexpr int kBlock = 256;                 // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kGroups = 2;                  // float4 groups per thread per tile
constexpr int kPerThread = 4 * kGroups;     // 8 elements per thread
constexpr int kTile = kBlock * kPerThread;  // 2048 elements per tile

// ------------------------------------------------------ exact fp32 ops
// Each is exactly one IEEE binary32 operation, round-to-nearest-even, never fused
// with a neighbour (the sign bits depend on this sequence bit for bit).
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float add_rn(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float sub_rn(float a, float b) { return __fsub_rn(a, b); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float f16_bits_to_float(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);  // exact widening
}

// Gradient element types: fp32, bf16, fp16 (the 16-bit ones widen exactly).
enum GradType { kGradF32 = 0, kGradBF16 = 1, kGradF16 = 2 };
template <int GT>
__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
    return GT == kGradBF16 ? bf16_bits_to_float(h16) : f16_bits_to_float(h16);
}

// binary32 -> bfloat16 bits, nearest-even; NaN kept quiet.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t round = 0x7fffu + ((u >> 16) & 1u);
    const uint32_t r = (u + round) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

// ------------------------------------------------- streaming accesses
// State that is read once and written once per call goes through nontemporal
// loads and stores (the streaming cache policy): on this GPU a kernel with five
// fp32 read streams and three write streams moves about 6% more bytes per second
// with both than with neither (either alone gives 1-2%).  Only where each access
// instruction of a wave covers whole contiguous cache lines: where the lanes of
// an instruction leave gaps (each thread owning 32 or 64 consecutive bytes and
// writing them 16 bytes at a time), streaming stores are far slower.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld_stream(const float4 *p) {
    const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2 *p) {
    const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t ld_stream(const uint32_t *p) { return __builtin_nontemporal_load(p); }
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t *>(p));
}
__device__ __forceinline__ void st_stream(float4 *p, float4 v) {
    const f32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t *>(p));
}
__device__ __forceinline__ void st_stream(uint2 *p, uint2 v) {
    const u32x2_t t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t *>(p));
}

// --------------------------------------------------------- double-double
// Error-free transformation a + b = s + err (Knuth's TwoSum); needs unfused fp64.
struct DD {
    double hi, lo;
};

__device__ __forceinline__ void two_sum(double a, double b, double &s, double &err) {
    s = __dadd_rn(a, b);
    const double bb = __dsub_rn(s, a);
    err = __dadd_rn(__dsub_rn(a, __dsub_rn(s, bb)), __dsub_rn(b, bb));
}

__device__ __forceinline__ void dd_add_term(DD &acc, double t) {
    double s, err;
    two_sum(acc.hi, t, s, err);
    acc.hi = s;
    acc.lo = __dadd_rn(acc.lo, err);
}

__device__ __forceinline__ DD dd_add(DD a, DD b) {
    double s, err;
    two_sum(a.hi, b.hi, s, err);
    const double lo = __dadd_rn(__dadd_rn(a.lo, b.lo), err);
    DD r;
    two_sum(s, lo, r.hi, r.lo);
    return r;
}

__device__ __forceinline__ double shfl_xor_d(double v, int mask) { return __shfl_xor(v, mask, 64); }

// Sum of a DD over the 64 lanes of a wave (butterfly; every lane gets the total).
__device__ __forceinline__ DD wave_sum_dd(DD v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        DD o;
        o.hi = shfl_xor_d(v.hi, m);
        o.lo = shfl_xor_d(v.lo, m);
        v = dd_add(v, o);
    }
    return v;
}

// ------------------------------------------------------- lane exchange
// OR over each aligned group of 8 lanes, via DPP: swap neighbours, swap pairs,
// then mirror inside the half-row of 8.
__device__ __forceinline__ uint32_t or_over_8_lanes(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return v;
}

// ------------------------------------------ single-location agent atomics
// Cross-workgroup traffic uses only these: relaxed, agent scope.  Every value a
// reader consumes is self-validating (an epoch tag or a tag bit), so no ordering
// between different addresses is ever relied on.
__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_agent(uint64_t *p, uint64_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t or_agent32(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged partial: the sign bit (never set in a sum of squares) marks "written".
constexpr uint64_t kTag = 1ull << 63;
__device__ __forceinline__ uint64_t tag_partial(double s) { return (uint64_t)__double_as_longlong(s) | kTag; }
__device__ __forceinline__ double untag_partial(uint64_t w) { return __longlong_as_double((long long)(w & ~kTag)); }

// ------------------------------------------------------------ Philox4x32-10
// Salmon et al., SC'11, sec. 4: per round two 32x32->64 products of counter words
// 0 and 2 with 0xD2511F53 / 0xCD9E8D57; the high halves are xored with counter
// words 3 / 1 and the round key; the key advances by 0x9E3779B9 / 0xBB67AE85.
struct U4 {
    uint32_t a, b, c, d;
};

__device__ __forceinline__ U4 philox4x32_10(U4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p = (uint64_t)ctr.a * 0xD2511F53u;
        const uint64_t q = (uint64_t)ctr.c * 0xCD9E8D57u;
        U4 nx;
        // three-input xors as one v_bitop3_b32 each (truth table 0x96 = odd parity)
        nx.a = __builtin_amdgcn_bitop3_b32((uint32_t)(q >> 32), ctr.b, k0, 0x96);
        nx.b = (uint32_t)q;
        nx.c = __builtin_amdgcn_bitop3_b32((uint32_t)(p >> 32), ctr.d, k1, 0x96);
        nx.d = (uint32_t)p;
        ctr = nx;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return ctr;
}

}  // namespace onebit

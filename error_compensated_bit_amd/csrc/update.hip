// update.hip -- the worker's finish after the compressed all-reduce (DeepSpeed
// 1-bit Adam guide, sec. 3.5 and sec. 4, phase two): the all-reduced momentum is
// multiplied by the per-element exp_avg_mask, then the parameters take the
// frozen-variance step x -= lr * (m / (sqrt(v) + eps) + weight_decay * x).
// Streaming; per element 12 bytes read and 4 written (x) without a mask, 13 read
// and 8 written with one (the masked momentum is stored back), plus 2 written for
// the optional bf16 copy of x.  Per group of four elements: one 128-bit access for
// each fp32 array, one 32-bit mask load, one 64-bit bf16 store.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace onebit {

// Groups of four elements per thread and iteration; group h of the threads of a
// workgroup covers 256 consecutive groups, so every access instruction of a wave
// covers whole contiguous cache lines (which the streaming cache policy needs).
constexpr int kUpdGroups = 2;

struct UpdateArgs {
    float *m;
    const uint8_t *mask;
    const float *v;
    float *x;
    uint16_t *xb;
    int64_t n;
    float lr, eps, wd;
};

__device__ __forceinline__ float finish_one(const UpdateArgs &a, float &m, uint32_t keep, float v, float x) {
    if (a.mask) m = mul_rn(m, keep ? 1.0f : 0.0f);
    const float upd = add_rn(m / (sqrtf(v) + a.eps), mul_rn(a.wd, x));
    return sub_rn(x, mul_rn(a.lr, upd));
}

template <bool MASK, bool XB>
__global__ __launch_bounds__(256) void k_momentum_update(UpdateArgs a) {
    const int64_t groups = a.n / 4;
    const int64_t span = (int64_t)blockDim.x * kUpdGroups;
    for (int64_t base = blockIdx.x * span; base < groups; base += (int64_t)gridDim.x * span) {
        float4 m4[kUpdGroups], v4[kUpdGroups], x4[kUpdGroups];
        uint32_t mk[kUpdGroups];
        bool in[kUpdGroups];
#pragma unroll
        for (int h = 0; h < kUpdGroups; ++h) {
            const int64_t q = base + h * (int64_t)blockDim.x + threadIdx.x;
            in[h] = q < groups;
            mk[h] = 0xffffffffu;
            if (in[h]) {
                m4[h] = ld_stream(reinterpret_cast<const float4 *>(a.m + 4 * q));
                v4[h] = ld_stream(reinterpret_cast<const float4 *>(a.v + 4 * q));
                x4[h] = ld_stream(reinterpret_cast<const float4 *>(a.x + 4 * q));
                if (MASK) mk[h] = ld_stream(reinterpret_cast<const uint32_t *>(a.mask + 4 * q));
            }
        }
#pragma unroll
        for (int h = 0; h < kUpdGroups; ++h) {
            if (!in[h]) continue;
            const int64_t q = base + h * (int64_t)blockDim.x + threadIdx.x;
            const uint32_t w = mk[h];
            float xn[4];
            xn[0] = finish_one(a, m4[h].x, w & 0xffu, v4[h].x, x4[h].x);
            xn[1] = finish_one(a, m4[h].y, (w >> 8) & 0xffu, v4[h].y, x4[h].y);
            xn[2] = finish_one(a, m4[h].z, (w >> 16) & 0xffu, v4[h].z, x4[h].z);
            xn[3] = finish_one(a, m4[h].w, w >> 24, v4[h].w, x4[h].w);
            if (MASK) st_stream(reinterpret_cast<float4 *>(a.m + 4 * q), m4[h]);
            st_stream(reinterpret_cast<float4 *>(a.x + 4 * q), make_float4(xn[0], xn[1], xn[2], xn[3]));
            if (XB) {
                uint2 pk;
                pk.x = float_to_bf16_bits(xn[0]) | (float_to_bf16_bits(xn[1]) << 16);
                pk.y = float_to_bf16_bits(xn[2]) | (float_to_bf16_bits(xn[3]) << 16);
                st_stream(reinterpret_cast<uint2 *>(a.xb + 4 * q), pk);
            }
        }
    }
    // ragged tail (n % 4 elements), one thread each
    const int64_t tail = a.n - 4 * groups;
    const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (gid < tail) {
        const int64_t i = 4 * groups + gid;
        float m = a.m[i];
        const float xn = finish_one(a, m, MASK ? a.mask[i] : 1u, a.v[i], a.x[i]);
        if (MASK) a.m[i] = m;
        a.x[i] = xn;
        if (XB) a.xb[i] = (uint16_t)float_to_bf16_bits(xn);
    }
}

// The finish with the all-reduced momentum in its compressed form: the server's
// sign words and chunk scales of a plan, m = +-scale times the mask (0 or 1).
// One 2048-element tile of the plan per workgroup and iteration, eight elements per
// thread as two groups of four (the layout of the compression kernels), so each
// thread's four signs sit in one word.  Nothing is written to m.
struct PackedUpdateArgs {
    const TileDesc *tiles;
    int64_t n_tiles;
    const uint32_t *m_bits;
    const float *m_scales;
    const uint8_t *mask;
    const float *v;
    float *x;
    uint16_t *xb;
    float lr, eps, wd;
};

template <bool XB>
__global__ __launch_bounds__(256) void k_momentum_update_packed(PackedUpdateArgs a) {
    for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const TileDesc t = a.tiles[tile];
        if (t.len == 0) continue;
        const float s = a.m_scales[t.chunk];
        const bool full = t.len == kTile && (t.start & 3) == 0;
#pragma unroll
        for (int r = 0; r < kGroups; ++r) {
            const uint32_t k0 = 4u * (threadIdx.x + kBlock * r);
            if (k0 >= (uint32_t)t.len) continue;
            const uint32_t nib = a.m_bits[t.word + (k0 >> 5)] >> (k0 & 31u);
            const int64_t i0 = t.start + k0;
            float m4[4], v4[4], x4[4], xn[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool in = k0 + q < (uint32_t)t.len;
                const bool keep = !a.mask || (in && a.mask[i0 + q] != 0);
                // as onebit_momentum_update forms it: m * (mask ? 1 : 0)
                m4[q] = mul_rn(((nib >> q) & 1u) ? -s : s, keep ? 1.0f : 0.0f);
            }
            if (full) {
                const float4 vv = ld_stream(reinterpret_cast<const float4 *>(a.v + i0));
                const float4 xx = ld_stream(reinterpret_cast<const float4 *>(a.x + i0));
                v4[0] = vv.x; v4[1] = vv.y; v4[2] = vv.z; v4[3] = vv.w;
                x4[0] = xx.x; x4[1] = xx.y; x4[2] = xx.z; x4[3] = xx.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bool in = k0 + q < (uint32_t)t.len;
                    v4[q] = in ? a.v[i0 + q] : 1.0f;
                    x4[q] = in ? a.x[i0 + q] : 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float upd = add_rn(m4[q] / (sqrtf(v4[q]) + a.eps), mul_rn(a.wd, x4[q]));
                xn[q] = sub_rn(x4[q], mul_rn(a.lr, upd));
            }
            if (full) {
                st_stream(reinterpret_cast<float4 *>(a.x + i0), make_float4(xn[0], xn[1], xn[2], xn[3]));
                if (XB) {
                    uint2 pk;
                    pk.x = float_to_bf16_bits(xn[0]) | (float_to_bf16_bits(xn[1]) << 16);
                    pk.y = float_to_bf16_bits(xn[2]) | (float_to_bf16_bits(xn[3]) << 16);
                    st_stream(reinterpret_cast<uint2 *>(a.xb + i0), pk);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < (uint32_t)t.len) {
                        a.x[i0 + q] = xn[q];
                        if (XB) a.xb[i0 + q] = (uint16_t)float_to_bf16_bits(xn[q]);
                    }
            }
        }
    }
}

// Decompression of a plan's sign words and chunk scales into fp32 (the
// all-gather-decompress of the compressed all-reduce): out = +-scale times the
// mask, with the tile layout of the packed finish.
struct DecompressArgs {
    const TileDesc *tiles;
    int64_t n_tiles;
    const uint32_t *bits;
    const float *scales;
    const uint8_t *mask;
    float *out;
};

__global__ __launch_bounds__(256) void k_decompress(DecompressArgs a) {
    for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const TileDesc t = a.tiles[tile];
        if (t.len == 0) continue;
        const float s = a.scales[t.chunk];
        const bool full = t.len == kTile && (t.start & 3) == 0;
#pragma unroll
        for (int r = 0; r < kGroups; ++r) {
            const uint32_t k0 = 4u * (threadIdx.x + kBlock * r);
            if (k0 >= (uint32_t)t.len) continue;
            const uint32_t nib = a.bits[t.word + (k0 >> 5)] >> (k0 & 31u);
            const int64_t i0 = t.start + k0;
            float o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool in = k0 + q < (uint32_t)t.len;
                const float mq = ((nib >> q) & 1u) ? -s : s;
                o[q] = a.mask ? mul_rn(mq, (in && a.mask[i0 + q] != 0) ? 1.0f : 0.0f) : mq;
            }
            if (full) {
                st_stream(reinterpret_cast<float4 *>(a.out + i0), make_float4(o[0], o[1], o[2], o[3]));
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < (uint32_t)t.len) a.out[i0 + q] = o[q];
            }
        }
    }
}

// The workers' full-precision gradient average of the warmup phase (the
// all-reduce, simulated over W rows in one GPU's memory): fp64 sum in worker order,
// one division by W, one rounding.  Four elements per thread and row per
// iteration, the rows' loads of a group issued before they are summed.
struct AverageArgs {
    const void *g;
    int64_t row_stride;
    int64_t n;
    int32_t W;
    double invW;  // 1 / W when W is a power of two (exact), else 0
    float *out;
};

template <int GT>
__device__ __forceinline__ void load_row4(const AverageArgs &a, int w, int64_t i0, bool full, double (&acc)[4]) {
    float f[4];
    if (full) {
        if (GT == kGradF32) {
            const float4 t = ld_stream(reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + w * a.row_stride + i0));
            f[0] = t.x; f[1] = t.y; f[2] = t.z; f[3] = t.w;
        } else {
            const uint2 t = ld_stream(reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.g) + w * a.row_stride + i0));
            f[0] = half_bits_to_float<GT>(t.x & 0xffffu);
            f[1] = half_bits_to_float<GT>(t.x >> 16);
            f[2] = half_bits_to_float<GT>(t.y & 0xffffu);
            f[3] = half_bits_to_float<GT>(t.y >> 16);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = i0 + q;
            f[q] = i < a.n ? (GT == kGradF32 ? static_cast<const float *>(a.g)[w * a.row_stride + i]
                                             : half_bits_to_float<GT>(static_cast<const uint16_t *>(a.g)[w * a.row_stride + i]))
                           : 0.0f;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __dadd_rn(acc[q], (double)f[q]);
}

template <int GT>
__global__ __launch_bounds__(256) void k_average_rows(AverageArgs a) {
    const int64_t groups = (a.n + 3) / 4;
    const bool vec = ((uintptr_t)a.g & 15u) == 0 && (a.row_stride & 3) == 0;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < groups; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i0 = 4 * q;
        const bool full = vec && i0 + 4 <= a.n;
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        for (int w = 0; w < a.W; ++w) load_row4<GT>(a, w, i0, full, acc);
        float o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = (float)(a.invW != 0.0 ? __dmul_rn(acc[k], a.invW) : __ddiv_rn(acc[k], (double)a.W));
        if (full) {
            st_stream(reinterpret_cast<float4 *>(a.out + i0), make_float4(o[0], o[1], o[2], o[3]));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i0 + k < a.n) a.out[i0 + k] = o[k];
        }
    }
}

static int64_t grid_for(int64_t work_items, int per_cu) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int64_t blocks = (work_items + 255) / 256;
    const int64_t cap = (int64_t)cus * per_cu;
    if (blocks > cap) blocks = cap;
    return blocks < 1 ? 1 : blocks;
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_decompress(onebit_plan_t plan, const uint32_t *bits, const float *scales,
                                             const uint8_t *mask, float *out, void *stream) {
    if (!plan) return ONEBIT_ERR_INVALID;
    if (plan->n == 0) return ONEBIT_OK;
    if (!bits || !scales || !out) return ONEBIT_ERR_INVALID;
    if (!aligned_to(bits, 4) || !aligned_to(scales, 4) || !aligned16(out)) return ONEBIT_ERR_ALIGN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;
    DecompressArgs a{plan->d_tiles, plan->n_tiles, bits, scales, mask, out};
    const int64_t blocks = std::min<int64_t>(plan->n_tiles, grid_for(plan->n_tiles * 256, 8));
    hipLaunchKernelGGL(k_decompress, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t onebit_average_rows(const void *g, onebit_dtype_t g_dtype, int W, int64_t row_stride,
                                               int64_t n, float *out, void *stream) {
    if (n < 0 || W < 1 || W > 65536) return ONEBIT_ERR_INVALID;
    if (g_dtype != ONEBIT_F32 && g_dtype != ONEBIT_BF16 && g_dtype != ONEBIT_F16) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!g || !out || (W > 1 && row_stride < n)) return ONEBIT_ERR_INVALID;
    if (!aligned16(out)) return ONEBIT_ERR_ALIGN;
    AverageArgs a{g, W > 1 ? row_stride : 0, n, W, (W & (W - 1)) == 0 ? 1.0 / (double)W : 0.0, out};
    const dim3 grid((unsigned)grid_for((n + 3) / 4, 8)), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (g_dtype == ONEBIT_BF16)
        hipLaunchKernelGGL(k_average_rows<kGradBF16>, grid, block, 0, s, a);
    else if (g_dtype == ONEBIT_F16)
        hipLaunchKernelGGL(k_average_rows<kGradF16>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(k_average_rows<kGradF32>, grid, block, 0, s, a);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t onebit_momentum_update_packed(onebit_plan_t plan, const uint32_t *m_bits,
                                                         const float *m_scales, const uint8_t *mask, const float *v,
                                                         float *x, uint16_t *x_bf16, double lr, double eps,
                                                         double weight_decay, void *stream) {
    if (!plan) return ONEBIT_ERR_INVALID;
    if (plan->n == 0) return ONEBIT_OK;
    if (!m_bits || !m_scales || !v || !x) return ONEBIT_ERR_INVALID;
    if (!aligned_to(m_bits, 4) || !aligned_to(m_scales, 4) || !aligned16(v) || !aligned16(x) ||
        (x_bf16 && !aligned16(x_bf16)))
        return ONEBIT_ERR_ALIGN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;
    PackedUpdateArgs a{};
    a.tiles = plan->d_tiles;
    a.n_tiles = plan->n_tiles;
    a.m_bits = m_bits;
    a.m_scales = m_scales;
    a.mask = mask;
    a.v = v;
    a.x = x;
    a.xb = x_bf16;
    a.lr = (float)lr;
    a.eps = (float)eps;
    a.wd = (float)weight_decay;
    int cus = 256;
    int v_cus = 0;
    if (hipDeviceGetAttribute(&v_cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_cus > 0)
        cus = v_cus;
    int64_t blocks = plan->n_tiles;
    const int64_t cap = (int64_t)cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    prof_before(kProfMomentumUpdate, s);
    if (x_bf16)
        hipLaunchKernelGGL(k_momentum_update_packed<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_momentum_update_packed<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    prof_after(s);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t onebit_momentum_update(float *m, const uint8_t *mask, const float *v, float *x,
                                                  uint16_t *x_bf16, int64_t n, double lr, double eps,
                                                  double weight_decay, void *stream) {
    if (n < 0) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!m || !v || !x) return ONEBIT_ERR_INVALID;
    if (!aligned16(m) || !aligned16(v) || !aligned16(x) || (mask && !aligned16(mask)) ||
        (x_bf16 && !aligned16(x_bf16)))
        return ONEBIT_ERR_ALIGN;
    UpdateArgs a{};
    a.m = m;
    a.mask = mask;
    a.v = v;
    a.x = x;
    a.xb = x_bf16;
    a.n = n;
    a.lr = (float)lr;
    a.eps = (float)eps;
    a.wd = (float)weight_decay;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_cus = 0;
        if (hipDeviceGetAttribute(&v_cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_cus > 0)
            cus = v_cus;
    }
    const int64_t groups = n / 4;
    int64_t blocks = (groups + 256 * kUpdGroups - 1) / (256 * kUpdGroups);
    const int64_t cap = (int64_t)cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(256);
    prof_before(kProfMomentumUpdate, s);
    if (mask && x_bf16)
        hipLaunchKernelGGL((k_momentum_update<true, true>), grid, block, 0, s, a);
    else if (mask)
        hipLaunchKernelGGL((k_momentum_update<true, false>), grid, block, 0, s, a);
    else if (x_bf16)
        hipLaunchKernelGGL((k_momentum_update<false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_momentum_update<false, false>), grid, block, 0, s, a);
    prof_after(s);
    return hip_status(hipGetLastError());
}

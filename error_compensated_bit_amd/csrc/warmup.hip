// warmup.hip -- full-precision Adam step of the warmup phase (DeepSpeed 1-bit Adam
// guide, sec. 4, phase one: standard first and second moments, full-precision
// gradients; sec. 3.4: lr, betas, eps, weight_decay, bias_correction).
// Pure streaming: 28 bytes per element with fp32 g (26 with bf16 g), 128-bit
// accesses, grid-stride over groups of four elements.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace onebit {

struct WarmupArgs {
    float *x, *m, *v;
    const void *g;
    int64_t n;
    float b1, ob1, b2, ob2, lr, eps, wd, bc1, bc2;
    int bias;
};

template <int GT>
__device__ __forceinline__ void warm_one(const WarmupArgs &a, float g, float &x, float &m, float &v) {
    m = add_rn(mul_rn(a.b1, m), mul_rn(a.ob1, g));
    v = add_rn(mul_rn(a.b2, v), mul_rn(a.ob2, mul_rn(g, g)));
    const float mh = a.bias ? m / a.bc1 : m;
    const float vh = a.bias ? v / a.bc2 : v;
    const float upd = mh / (sqrtf(vh) + a.eps) + a.wd * x;
    x = x - a.lr * upd;
}

template <int GT>
__device__ __forceinline__ void load_g4w(const void *g, int64_t i, float (&gg)[4]) {
    if (GT != kGradF32) {
        const uint2 h = ld_stream(reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(g) + i));
        gg[0] = half_bits_to_float<GT>(h.x & 0xffffu);
        gg[1] = half_bits_to_float<GT>(h.x >> 16);
        gg[2] = half_bits_to_float<GT>(h.y & 0xffffu);
        gg[3] = half_bits_to_float<GT>(h.y >> 16);
    } else {
        const float4 h = ld_stream(reinterpret_cast<const float4 *>(static_cast<const float *>(g) + i));
        gg[0] = h.x; gg[1] = h.y; gg[2] = h.z; gg[3] = h.w;
    }
}

// Each thread takes kWU groups of four elements per iteration (all loads of an
// iteration in flight together, 512 bytes per thread), grid-stride over the
// vector.  Measured on the 335M-element vector: kWU 2 / 4 / 8 / 16 run at 4.8 /
// 5.3 / 5.5 / 5.0 TB/s (16 needs ~370 VGPRs).
constexpr int kWU = 8;

template <int GT>
__global__ __launch_bounds__(256) void k_adam_warmup(WarmupArgs a) {
    const int64_t groups = a.n / 4;
    const int64_t span = (int64_t)blockDim.x * kWU;
    for (int64_t base = blockIdx.x * span; base < groups; base += (int64_t)gridDim.x * span) {
        float gg[kWU][4];
        float4 xx[kWU], mm[kWU], vv[kWU];
        bool in[kWU];
#pragma unroll
        for (int u = 0; u < kWU; ++u) {
            const int64_t q = base + u * (int64_t)blockDim.x + threadIdx.x;
            in[u] = q < groups;
            if (in[u]) {
                load_g4w<GT>(a.g, 4 * q, gg[u]);
                xx[u] = ld_stream(reinterpret_cast<const float4 *>(a.x + 4 * q));
                mm[u] = ld_stream(reinterpret_cast<const float4 *>(a.m + 4 * q));
                vv[u] = ld_stream(reinterpret_cast<const float4 *>(a.v + 4 * q));
            }
        }
#pragma unroll
        for (int u = 0; u < kWU; ++u) {
            if (!in[u]) continue;
            const int64_t q = base + u * (int64_t)blockDim.x + threadIdx.x;
            warm_one<GT>(a, gg[u][0], xx[u].x, mm[u].x, vv[u].x);
            warm_one<GT>(a, gg[u][1], xx[u].y, mm[u].y, vv[u].y);
            warm_one<GT>(a, gg[u][2], xx[u].z, mm[u].z, vv[u].z);
            warm_one<GT>(a, gg[u][3], xx[u].w, mm[u].w, vv[u].w);
            st_stream(reinterpret_cast<float4 *>(a.x + 4 * q), xx[u]);
            st_stream(reinterpret_cast<float4 *>(a.m + 4 * q), mm[u]);
            st_stream(reinterpret_cast<float4 *>(a.v + 4 * q), vv[u]);
        }
    }
    // ragged tail (n % 4 elements), one thread each
    const int64_t tail = a.n - 4 * groups;
    const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (gid < tail) {
        const int64_t i = 4 * groups + gid;
        const float g = GT != kGradF32 ? half_bits_to_float<GT>(static_cast<const uint16_t *>(a.g)[i])
                                       : static_cast<const float *>(a.g)[i];
        float x = a.x[i], m = a.m[i], v = a.v[i];
        warm_one<GT>(a, g, x, m, v);
        a.x[i] = x;
        a.m[i] = m;
        a.v[i] = v;
    }
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_adam_warmup_step(float *x, float *m, float *v, const void *g,
                                                   onebit_dtype_t g_dtype, int64_t n, double lr, double beta1,
                                                   double beta2, double eps, double weight_decay,
                                                   int bias_correction, int64_t step, void *stream) {
    if (n < 0 || step < 1) return ONEBIT_ERR_INVALID;
    if (g_dtype != ONEBIT_F32 && g_dtype != ONEBIT_BF16 && g_dtype != ONEBIT_F16) return ONEBIT_ERR_INVALID;
    if (n == 0) return ONEBIT_OK;
    if (!x || !m || !v || !g) return ONEBIT_ERR_INVALID;
    if (!aligned16(x) || !aligned16(m) || !aligned16(v) || !aligned16(g)) return ONEBIT_ERR_ALIGN;
    WarmupArgs a{};
    a.x = x;
    a.m = m;
    a.v = v;
    a.g = g;
    a.n = n;
    a.b1 = (float)beta1;
    a.ob1 = (float)(1.0 - beta1);
    a.b2 = (float)beta2;
    a.ob2 = (float)(1.0 - beta2);
    a.lr = (float)lr;
    a.eps = (float)eps;
    a.wd = (float)weight_decay;
    a.bias = bias_correction ? 1 : 0;
    a.bc1 = bias_correction ? (float)(1.0 - pow(beta1, (double)step)) : 1.0f;
    a.bc2 = bias_correction ? (float)(1.0 - pow(beta2, (double)step)) : 1.0f;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v_cus = 0;
        if (hipDeviceGetAttribute(&v_cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v_cus > 0)
            cus = v_cus;
    }
    const int64_t groups = n / 4;
    int64_t blocks = (groups + 256 * kWU - 1) / (256 * kWU);
    const int64_t cap = (int64_t)cus * 6;  // six workgroups per CU: enough bytes in flight, fewer DRAM page conflicts
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    prof_before(kProfWarmup, s);
    if (g_dtype == ONEBIT_BF16)
        hipLaunchKernelGGL(k_adam_warmup<kGradBF16>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else if (g_dtype == ONEBIT_F16)
        hipLaunchKernelGGL(k_adam_warmup<kGradF16>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_adam_warmup<kGradF32>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    prof_after(s);
    return hip_status(hipGetLastError());
}

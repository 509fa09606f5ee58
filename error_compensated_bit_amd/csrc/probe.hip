// probe.hip -- a plain streaming kernel that measures what HBM delivers for a given
// mix of fp32 read and write streams on this device (diagnostics: the compression
// kernels are compared against it).  Each thread moves four 16-byte vectors of
// every stream per iteration, grid-stride, through the streaming cache policy the
// compression kernels use; out_k = sum of the inputs + k, so no stream can be
// elided.
#include "device_common.h"
#include "internal.h"

namespace onebit {

constexpr int kProbeU = 4;

template <int R, int WR>
__global__ __launch_bounds__(1024) void k_stream_probe(const float4 *const *in, float4 *const *out, int64_t n4) {
    const float4 *src[R];
    float4 *dst[WR];
#pragma unroll
    for (int r = 0; r < R; ++r) src[r] = in[r];
#pragma unroll
    for (int w = 0; w < WR; ++w) dst[w] = out[w];
    const int64_t span = (int64_t)blockDim.x * kProbeU;
    for (int64_t base = blockIdx.x * span; base < n4; base += (int64_t)gridDim.x * span) {
        float4 acc[kProbeU];
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int u = 0; u < kProbeU; ++u) {
                const int64_t i = base + u * (int64_t)blockDim.x + threadIdx.x;
                if (i < n4) {
                    const float4 v = ld_stream(src[r] + i);
                    acc[u].x += v.x; acc[u].y += v.y; acc[u].z += v.z; acc[u].w += v.w;
                }
            }
        }
#pragma unroll
        for (int w = 0; w < WR; ++w) {
#pragma unroll
            for (int u = 0; u < kProbeU; ++u) {
                const int64_t i = base + u * (int64_t)blockDim.x + threadIdx.x;
                const float k = (float)w;
                if (i < n4) st_stream(dst[w] + i, make_float4(acc[u].x + k, acc[u].y + k, acc[u].z + k, acc[u].w + k));
            }
        }
    }
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_stream_probe(const float *const *in, int reads, float *const *out, int writes,
                                               int64_t n, int grid, int block, void *stream) {
    if (n < 0 || grid < 1 || !in || !out) return ONEBIT_ERR_INVALID;
    if (block != 256 && block != 512 && block != 1024) return ONEBIT_ERR_INVALID;
    if (n % 4 != 0) return ONEBIT_ERR_ALIGN;
    const bool five_three = reads == 5 && writes == 3, one_one = reads == 1 && writes == 1;
    if (!five_three && !one_one) return ONEBIT_ERR_UNSUPPORTED;
    if (n == 0) return ONEBIT_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const auto *i4 = reinterpret_cast<const float4 *const *>(in);
    auto *o4 = reinterpret_cast<float4 *const *>(out);
    if (five_three)
        hipLaunchKernelGGL((k_stream_probe<5, 3>), dim3(grid), dim3(block), 0, s, i4, o4, n / 4);
    else
        hipLaunchKernelGGL((k_stream_probe<1, 1>), dim3(grid), dim3(block), 0, s, i4, o4, n / 4);
    return hip_status(hipGetLastError());
}

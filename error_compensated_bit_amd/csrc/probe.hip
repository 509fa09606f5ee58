// probe.hip -- a plain streaming kernel that measures what HBM delivers for a given
// mix of fp32 read and write streams on this device (diagnostics: the compression
// kernels are compared against it).  Each thread moves four 16-byte vectors of
// every stream per iteration, grid-stride, through either the streaming
// (nontemporal) cache policy the compression kernels use or the default policy;
// out_k = sum of the inputs + k, so no stream can be elided.  With no output
// stream the sum is stored back into the first input only where it equals a value
// that sums of the probe's zero-filled inputs never take, so the loads stay live
// and nothing is written.
#include "device_common.h"
#include "internal.h"

namespace onebit {

constexpr int kProbeU = 4;

template <bool NT>
__device__ __forceinline__ float4 probe_load(const float4 *p) {
    if (NT) return ld_stream(p);
    return *p;
}
template <bool NT>
__device__ __forceinline__ void probe_store(float4 *p, float4 v) {
    if (NT)
        st_stream(p, v);
    else
        *p = v;
}

template <int R, int WR, bool NT>
__global__ __launch_bounds__(1024) void k_stream_probe(const float4 *const *in, float4 *const *out, int64_t n4) {
    const float4 *src[R > 0 ? R : 1];
    float4 *dst[WR > 0 ? WR : 1];
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
                    const float4 v = probe_load<NT>(src[r] + i);
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
                if (i < n4)
                    probe_store<NT>(dst[w] + i, make_float4(acc[u].x + k, acc[u].y + k, acc[u].z + k, acc[u].w + k));
            }
        }
        if constexpr (WR == 0 && R > 0) {
#pragma unroll
            for (int u = 0; u < kProbeU; ++u) {
                const int64_t i = base + u * (int64_t)blockDim.x + threadIdx.x;
                if (i < n4 && acc[u].x == -3.0e38f) const_cast<float4 *>(src[0])[i] = acc[u];
            }
        }
    }
}

template <int R, int WR>
static void launch_probe(bool nt, const float4 *const *in, float4 *const *out, int64_t n4, int grid, int block,
                         hipStream_t s) {
    if (nt)
        hipLaunchKernelGGL((k_stream_probe<R, WR, true>), dim3(grid), dim3(block), 0, s, in, out, n4);
    else
        hipLaunchKernelGGL((k_stream_probe<R, WR, false>), dim3(grid), dim3(block), 0, s, in, out, n4);
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_stream_probe(const float *const *in, int reads, float *const *out, int writes,
                                               int64_t n, int grid, int block, int nontemporal, void *stream) {
    if (n < 0 || grid < 1 || (reads > 0 && !in) || (writes > 0 && !out)) return ONEBIT_ERR_INVALID;
    if (block != 256 && block != 512 && block != 1024) return ONEBIT_ERR_INVALID;
    if (n % 4 != 0) return ONEBIT_ERR_ALIGN;
    const int mix = reads * 10 + writes;
    switch (mix) {
        case 10: case 1: case 11: case 21: case 31: case 12: case 22: case 42: case 53: break;
        default: return ONEBIT_ERR_UNSUPPORTED;
    }
    if (n == 0) return ONEBIT_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const auto *i4 = reinterpret_cast<const float4 *const *>(in);
    auto *o4 = reinterpret_cast<float4 *const *>(out);
    const bool nt = nontemporal != 0;
    const int64_t n4 = n / 4;
    switch (mix) {
        case 10: launch_probe<1, 0>(nt, i4, o4, n4, grid, block, s); break;
        case 1: launch_probe<0, 1>(nt, i4, o4, n4, grid, block, s); break;
        case 11: launch_probe<1, 1>(nt, i4, o4, n4, grid, block, s); break;
        case 21: launch_probe<2, 1>(nt, i4, o4, n4, grid, block, s); break;
        case 31: launch_probe<3, 1>(nt, i4, o4, n4, grid, block, s); break;
        case 12: launch_probe<1, 2>(nt, i4, o4, n4, grid, block, s); break;
        case 22: launch_probe<2, 2>(nt, i4, o4, n4, grid, block, s); break;
        case 42: launch_probe<4, 2>(nt, i4, o4, n4, grid, block, s); break;
        default: launch_probe<5, 3>(nt, i4, o4, n4, grid, block, s); break;
    }
    return hip_status(hipGetLastError());
}

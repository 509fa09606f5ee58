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

// The same streams with the loads staged in LDS by the load unit itself (gfx950's
// 16-byte global-to-LDS loads, streaming policy): every wave double-buffers its own
// chunk of kProbeLdsU x 64 float4 per input stream, issuing the next chunk's loads
// before it reads the current chunk back, so the bytes in flight hold no VGPRs.
// Each wave reads only what it loaded itself, so no workgroup barrier is needed;
// the wait for a chunk counts the wave's own outstanding vector-memory operations,
// which complete in issue order, and leaves the next chunk's loads and the previous
// chunk's stores in flight.  256-thread workgroups.
constexpr int kProbeLdsU = 4;
constexpr int kProbeLdsWaves = 4;
constexpr int kAuxNontemporal = 2;          // cache-policy operand of the LDS load: nt

template <int R>
struct ProbeStage {
    float4 v[R][kProbeLdsU][kProbeLdsWaves][64];
};

// s_waitcnt with vmcnt = n (n < 64) and no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int R>
__device__ __forceinline__ void probe_issue(const float4 *const *src, ProbeStage<R> &st, int64_t c, int64_t n4,
                                            int wave, int lane) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int u = 0; u < kProbeLdsU; ++u) {
            int64_t i = (c * kProbeLdsU + u) * 64 + lane;
            if (i >= n4) i = n4 - 1;            // an in-bounds address; the value is not used
            __builtin_amdgcn_global_load_lds(src[r] + i,
                                             (__attribute__((address_space(3))) void *)&st.v[r][u][wave][0], 16,
                                             0, kAuxNontemporal);
        }
    }
}

typedef float lds_f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) lds_f32x4_t *global_f32x4_ptr;

// One 16-byte LDS read, complete when the asm block ends.  Written as asm so that
// the compiler's wait insertion, which cannot tell the two stages apart, does not
// wait for every outstanding global-to-LDS load before it; the stage being read was
// waited for by its vmcnt count.
__device__ __forceinline__ lds_f32x4_t lds_read16(const float4 *p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
    lds_f32x4_t v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}

template <int R, int WR>
__device__ __forceinline__ void probe_finish(const ProbeStage<R> &st, const float4 *const *src, float4 *const *dst,
                                             int64_t c, int64_t n4, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < kProbeLdsU; ++u) {
        const int64_t i = (c * kProbeLdsU + u) * 64 + lane;
        lds_f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const lds_f32x4_t v = lds_read16(&st.v[r][u][wave][lane]);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        // stores through global pointers: a flat store could reach LDS, and the
        // compiler would wait for the global-to-LDS loads in flight before it
#pragma unroll
        for (int w = 0; w < WR; ++w) {
            const float k = (float)w;
            const lds_f32x4_t o = {acc.x + k, acc.y + k, acc.z + k, acc.w + k};
            if (i < n4) __builtin_nontemporal_store(o, (global_f32x4_ptr)(dst[w] + i));
        }
        if constexpr (WR == 0) {
            if (i < n4 && acc.x == -3.0e38f) {
                *(global_f32x4_ptr)(const_cast<float4 *>(src[0]) + i) = acc;
                wait_vm<0>();       // keeps the count of the wave's outstanding operations exact
            }
        }
    }
}

template <int R, int WR>
__global__ __launch_bounds__(256) void k_stream_probe_lds(const float4 *const *in, float4 *const *out, int64_t n4) {
    __shared__ ProbeStage<R> s0, s1;
    const float4 *src[R];
    float4 *dst[WR > 0 ? WR : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) src[r] = in[r];
#pragma unroll
    for (int w = 0; w < WR; ++w) dst[w] = out[w];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t chunks = (n4 + kProbeLdsU * 64 - 1) / (kProbeLdsU * 64);
    const int64_t stride = (int64_t)gridDim.x * kProbeLdsWaves;
    constexpr int kLoads = R * kProbeLdsU, kStores = WR * kProbeLdsU;
    int64_t c = (int64_t)blockIdx.x * kProbeLdsWaves + wave;
    if (c >= chunks) return;
    probe_issue<R>(src, s0, c, n4, wave, lane);
    bool first = true;
    while (true) {
        // chunk c is in s0; the next one goes to s1
        const int64_t c1 = c + stride;
        if (c1 < chunks) {
            probe_issue<R>(src, s1, c1, n4, wave, lane);
            if (first) wait_vm<kLoads>(); else wait_vm<kLoads + kStores>();
        } else {
            if (first) wait_vm<0>(); else wait_vm<kStores>();
        }
        first = false;
        probe_finish<R, WR>(s0, src, dst, c, n4, wave, lane);
        if (c1 >= chunks) break;
        // chunk c1 is in s1; the next one goes to s0
        const int64_t c2 = c1 + stride;
        if (c2 < chunks) {
            probe_issue<R>(src, s0, c2, n4, wave, lane);
            wait_vm<kLoads + kStores>();
        } else {
            wait_vm<kStores>();
        }
        probe_finish<R, WR>(s1, src, dst, c1, n4, wave, lane);
        if (c2 >= chunks) break;
        c = c2;
    }
}

template <int R, int WR>
static void launch_probe(int policy, const float4 *const *in, float4 *const *out, int64_t n4, int grid, int block,
                         hipStream_t s) {
    if (policy == 2) {
        if constexpr (R > 0)
            hipLaunchKernelGGL((k_stream_probe_lds<R, WR>), dim3(grid), dim3(block), 0, s, in, out, n4);
    } else if (policy == 1) {
        hipLaunchKernelGGL((k_stream_probe<R, WR, true>), dim3(grid), dim3(block), 0, s, in, out, n4);
    } else {
        hipLaunchKernelGGL((k_stream_probe<R, WR, false>), dim3(grid), dim3(block), 0, s, in, out, n4);
    }
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_stream_probe(const float *const *in, int reads, float *const *out, int writes,
                                               int64_t n, int grid, int block, int policy, void *stream) {
    if (n < 0 || grid < 1 || (reads > 0 && !in) || (writes > 0 && !out)) return ONEBIT_ERR_INVALID;
    if (block != 256 && block != 512 && block != 1024) return ONEBIT_ERR_INVALID;
    if (policy < 0 || policy > 2 || (policy == 2 && (block != 256 || reads == 0))) return ONEBIT_ERR_INVALID;
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
    const int64_t n4 = n / 4;
    switch (mix) {
        case 10: launch_probe<1, 0>(policy, i4, o4, n4, grid, block, s); break;
        case 1: launch_probe<0, 1>(policy, i4, o4, n4, grid, block, s); break;
        case 11: launch_probe<1, 1>(policy, i4, o4, n4, grid, block, s); break;
        case 21: launch_probe<2, 1>(policy, i4, o4, n4, grid, block, s); break;
        case 31: launch_probe<3, 1>(policy, i4, o4, n4, grid, block, s); break;
        case 12: launch_probe<1, 2>(policy, i4, o4, n4, grid, block, s); break;
        case 22: launch_probe<2, 2>(policy, i4, o4, n4, grid, block, s); break;
        case 42: launch_probe<4, 2>(policy, i4, o4, n4, grid, block, s); break;
        default: launch_probe<5, 3>(policy, i4, o4, n4, grid, block, s); break;
    }
    return hip_status(hipGetLastError());
}

// ------------------------------------------------------------ Philox probe
// The random numbers of the quantizers alone: thread t of the grid draws the
// Philox4x32-10 blocks t, t + T, t + 2T, ... below n_blocks (T = threads in the
// grid; counter = block index, key = the seed's two words, as the quantizers draw
// them) and folds the four words of every block into one word by XOR, stored to
// out[t].  One block serves four quantized elements.
namespace onebit {

__global__ __launch_bounds__(1024) void k_philox_probe(uint32_t k0, uint32_t k1, int64_t n_blocks, uint32_t *out) {
    const int64_t T = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (int64_t blk = t; blk < n_blocks; blk += T) {
        const U4 r = philox4x32_10(U4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u}, k0, k1);
        acc ^= r.a ^ r.b ^ r.c ^ r.d;
    }
    out[t] = acc;
}

}  // namespace onebit

extern "C" onebit_status_t onebit_philox_probe(uint64_t seed, int64_t n_blocks, uint32_t *out, int grid, int block,
                                               void *stream) {
    if (n_blocks < 0 || grid < 1 || !out) return ONEBIT_ERR_INVALID;
    if (block != 256 && block != 512 && block != 1024) return ONEBIT_ERR_INVALID;
    hipLaunchKernelGGL(k_philox_probe, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream),
                       (uint32_t)seed, (uint32_t)(seed >> 32), n_blocks, out);
    return hip_status(hipGetLastError());
}

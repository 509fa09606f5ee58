// compress.hip -- the error-compensated 1-bit compression step of 1-bit Adam on
// gfx950: worker compression fused with the frozen-v update, and the server stage
// of the compressed all-reduce.
//
// What is computed (DeepSpeed 1-bit Adam guide, sec. 4 and sec. 3.5; 1-bit Adam
// review, "proposed method"):  per element m1 = b1 m + (1-b1) g, c = m1 + e; per
// chunk one scale sqrt(sum c^2)/sqrt(n_chunk); per element one sign bit (c < 0),
// q = +-scale, e = c - q, m = q (0 for masked tensors, with e = 0), and the
// preconditioned step x -= lr (m / (sqrt(v) + eps) + wd x) with v frozen.
//
// How: the flat vector is cut into tiles of 4096 elements (256 threads x 16).
// A tile computes its c into registers, writes its sign words, and posts its
// fp64 partial sum of squares.  The chunk scale needs every tile of the chunk, so
//  - chunks of at most R tiles (R = co-resident workgroups) are done in ONE pass
//    by a cooperative persistent kernel: each tile keeps c in registers, waits for
//    its chunk's scale, then finishes -- HBM sees each input once and each output
//    once;
//  - larger chunks take two passes: pass 1 stores c in place of e, pass 2 reads it
//    back with v and x once the chunk scale is known.
// Cross-workgroup communication uses only single-location relaxed agent-scope
// atomics on self-validating words (tagged partials, {epoch, count} and
// {epoch, scale}); no cache-wide write-back or invalidate is ever needed, and a
// zeroed workspace is always ready for the next call.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace onebit {

enum Mode { kUpdate = 0, kCompressOnly = 1, kServer = 2 };

struct CompressArgs {
    const TileDesc *tiles;
    const ChunkDesc *chunks;
    const int64_t *mask_iv;
    const int32_t *list;
    int32_t list_len;
    int32_t aligned;
    // worker inputs / state
    const void *g;
    float *m;
    float *e;         // worker error, or the server error in server mode
    const float *v;
    float *x;
    uint16_t *xb;
    // server inputs
    const uint32_t *wbits;
    const float *wscales;
    int32_t W;
    int64_t plan_words;
    int64_t n_chunks;
    float *m_out;
    // outputs
    uint32_t *bits;
    float *scales;
    // hyperparameters (binary32)
    float b1, ob1, lr, eps, wd;
    // workspace
    uint64_t *err;
    uint64_t *chunk_words;
    uint64_t *slots;
    uint32_t spin_limit;
};

// Bound of every cross-workgroup wait (iterations of a short sleep and a reload).
// A wait that runs out records an error in the workspace; from then on no wait
// of any workgroup spins again, so a kernel always drains in bounded time.
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ bool give_up(const CompressArgs &a, uint32_t spins) {
    return spins >= a.spin_limit || ((spins & 255u) == 255u && ld_agent(a.err) != 0);
}

// ---------------------------------------------------------------- tile: c
template <int MODE, bool GBF16>
__device__ __forceinline__ void tile_compute_c(const CompressArgs &a, const TileDesc &t,
                                               float (&c)[kPerThread], const double *s_wscale) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const int k0 = 4 * (tid + kBlock * r);
        const int64_t i0 = t.start + k0;
        if (MODE != kServer) {
            float g4[4], m4[4], e4[4];
            if (a.aligned && k0 + 3 < t.len) {
                if (GBF16) {
                    const uint2 gg = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.g) + i0);
                    g4[0] = bf16_bits_to_float(gg.x & 0xffffu);
                    g4[1] = bf16_bits_to_float(gg.x >> 16);
                    g4[2] = bf16_bits_to_float(gg.y & 0xffffu);
                    g4[3] = bf16_bits_to_float(gg.y >> 16);
                } else {
                    const float4 gg = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.g) + i0);
                    g4[0] = gg.x; g4[1] = gg.y; g4[2] = gg.z; g4[3] = gg.w;
                }
                const float4 mm = *reinterpret_cast<const float4 *>(a.m + i0);
                const float4 ee = *reinterpret_cast<const float4 *>(a.e + i0);
                m4[0] = mm.x; m4[1] = mm.y; m4[2] = mm.z; m4[3] = mm.w;
                e4[0] = ee.x; e4[1] = ee.y; e4[2] = ee.z; e4[3] = ee.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bool in = k0 + q < t.len;
                    const int64_t i = i0 + q;
                    g4[q] = in ? (GBF16 ? bf16_bits_to_float(static_cast<const uint16_t *>(a.g)[i])
                                        : static_cast<const float *>(a.g)[i])
                               : 0.0f;
                    m4[q] = in ? a.m[i] : 0.0f;
                    e4[q] = in ? a.e[i] : 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float m1 = add_rn(mul_rn(a.b1, m4[q]), mul_rn(a.ob1, g4[q]));
                c[4 * r + q] = (k0 + q < t.len) ? add_rn(m1, e4[q]) : 0.0f;
            }
        } else {
            // server: average of the W workers' decompressed values, fp64 in worker order
            double acc[4] = {0.0, 0.0, 0.0, 0.0};
            if (k0 < t.len) {
                const int64_t word = t.word + (k0 >> 5);
                const int sh = k0 & 31;
                for (int w = 0; w < a.W; ++w) {
                    const uint32_t bw = a.wbits[(int64_t)w * a.plan_words + word] >> sh;
                    const double s = s_wscale[w];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = __dadd_rn(acc[q], ((bw >> q) & 1u) ? -s : s);
                }
            }
            float es[4];
            if (a.aligned && k0 + 3 < t.len) {
                const float4 ee = *reinterpret_cast<const float4 *>(a.e + i0);
                es[0] = ee.x; es[1] = ee.y; es[2] = ee.z; es[3] = ee.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) es[q] = (k0 + q < t.len) ? a.e[i0 + q] : 0.0f;
            }
            const double dW = (double)a.W;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float avg = (float)__ddiv_rn(acc[q], dW);
                c[4 * r + q] = (k0 + q < t.len) ? add_rn(avg, es[q]) : 0.0f;
            }
        }
    }
}

// ------------------------------------------------------- tile: sign words
__device__ __forceinline__ void tile_store_bits(const CompressArgs &a, const TileDesc &t,
                                                const float (&c)[kPerThread]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const int k0 = 4 * (tid + kBlock * r);
        uint32_t nib = (c[4 * r + 0] < 0.0f ? 1u : 0u) | (c[4 * r + 1] < 0.0f ? 2u : 0u) |
                       (c[4 * r + 2] < 0.0f ? 4u : 0u) | (c[4 * r + 3] < 0.0f ? 8u : 0u);
        const uint32_t word = or_over_8_lanes(nib << (k0 & 31));
        if ((tid & 7) == 0 && k0 < t.len) a.bits[t.word + (k0 >> 5)] = word;
    }
}

// --------------------------------------------- tile: partial sum of squares
// Every square is exact in fp64; per-thread and cross-lane sums are double-double,
// and the tile's total is rounded to one fp64 value.
__device__ __forceinline__ double tile_sum_squares(const float (&c)[kPerThread], DD *s_red) {
    DD acc = {0.0, 0.0};
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const double cj = (double)c[j];
        dd_add_term(acc, __dmul_rn(cj, cj));
    }
    acc = wave_sum_dd(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_red[wave] = acc;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0) {
        DD t = s_red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t = dd_add(t, s_red[w]);
        total = __dadd_rn(t.hi, t.lo);
    }
    __syncthreads();  // s_red is reused by the caller
    return total;     // meaningful in thread 0 only
}

__device__ __forceinline__ void spin_pause() { __builtin_amdgcn_s_sleep(2); }

// The last tile of a chunk to arrive sums the chunk's partials (in tile order, so
// the result does not depend on arrival order), publishes the scale, and leaves
// the chunk's words and slots ready for the next call.
__device__ float finalize_chunk(const CompressArgs &a, int chunk, uint32_t epoch, DD *s_red) {
    const ChunkDesc ch = a.chunks[chunk];
    DD acc = {0.0, 0.0};
    for (int k = threadIdx.x; k < ch.ntiles; k += kBlock) {
        uint64_t *slot = a.slots + ch.first_tile + k;
        uint64_t w = ld_agent(slot);
        uint32_t spins = 0;
        while (!(w & kTag) && !give_up(a, spins)) {
            spin_pause();
            w = ld_agent(slot);
            ++spins;
        }
        if (!(w & kTag)) st_agent(a.err, 1);
        dd_add_term(acc, untag_partial(w));
        st_agent(slot, 0);
    }
    acc = wave_sum_dd(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_red[wave] = acc;
    __syncthreads();
    float scale = 0.0f;
    if (threadIdx.x == 0) {
        DD t = s_red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t = dd_add(t, s_red[w]);
        const double S = __dadd_rn(t.hi, t.lo);
        scale = ch.len > 0 ? (float)__ddiv_rn(__dsqrt_rn(S), __dsqrt_rn((double)ch.len)) : 0.0f;
        a.scales[chunk] = scale;
        const uint64_t next = (uint64_t)(uint32_t)(epoch + 1u) << 32;
        st_agent(a.chunk_words + 2 * chunk + 1, next | (uint64_t)__float_as_uint(scale));
        st_agent(a.chunk_words + 2 * chunk + 0, next);
    }
    __syncthreads();
    return scale;  // meaningful in thread 0 only
}

// Post this tile's partial and arrive.  WAIT: block until the chunk scale is
// published (one-pass path); otherwise return after arriving (pass 1 of two).
template <bool WAIT>
__device__ float arrive(const CompressArgs &a, int tile_id, int chunk, double partial, DD *s_red,
                        float *s_scale, uint32_t *s_flag) {
    if (threadIdx.x == 0) {
        st_agent(a.slots + tile_id, tag_partial(partial));
        const uint64_t old = add_agent(a.chunk_words + 2 * chunk, 1);
        const uint32_t epoch = (uint32_t)(old >> 32);
        const uint32_t count = (uint32_t)old;
        s_flag[0] = (count + 1u == (uint32_t)a.chunks[chunk].ntiles) ? 1u : 0u;
        s_flag[1] = epoch;
    }
    __syncthreads();
    const bool last = s_flag[0] != 0;
    const uint32_t epoch = s_flag[1];
    float scale = 0.0f;
    if (last) {
        scale = finalize_chunk(a, chunk, epoch, s_red);
        if (threadIdx.x == 0) *s_scale = scale;
    } else if (WAIT) {
        if (threadIdx.x == 0) {
            const uint64_t *pub = a.chunk_words + 2 * chunk + 1;
            const uint32_t want = epoch + 1u;
            uint64_t w = ld_agent(pub);
            uint32_t spins = ld_agent(a.err) != 0 ? a.spin_limit : 0u;
            while ((uint32_t)(w >> 32) != want && !give_up(a, spins)) {
                spin_pause();
                w = ld_agent(pub);
                ++spins;
            }
            if ((uint32_t)(w >> 32) != want) st_agent(a.err, 2);
            *s_scale = __uint_as_float((uint32_t)w);
        }
    }
    __syncthreads();
    scale = *s_scale;
    __syncthreads();
    return scale;
}

__device__ __forceinline__ bool masked_at(const CompressArgs &a, const TileDesc &t, int64_t i) {
    bool mk = false;
    for (int k = t.mask_lo; k < t.mask_hi; ++k) mk |= (i >= a.mask_iv[2 * k]) && (i < a.mask_iv[2 * k + 1]);
    return mk;
}

// ------------------------------------------------------- tile: finish
template <int MODE, bool XB>
__device__ __forceinline__ void tile_finish(const CompressArgs &a, const TileDesc &t,
                                            const float (&c)[kPerThread], float scale) {
    const int tid = threadIdx.x;
    const bool all_masked = t.mask_lo < 0;
    const bool some_masked = t.mask_hi > t.mask_lo;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const int k0 = 4 * (tid + kBlock * r);
        const int64_t i0 = t.start + k0;
        float q4[4], e4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float cq = c[4 * r + q];
            q4[q] = cq < 0.0f ? -scale : scale;
            e4[q] = sub_rn(cq, q4[q]);
            if (MODE != kServer) {
                const bool mk = all_masked || (some_masked && masked_at(a, t, i0 + q));
                if (mk) {
                    q4[q] = 0.0f;
                    e4[q] = 0.0f;
                }
            }
        }
        const bool full = a.aligned && k0 + 3 < t.len;
        if (MODE == kServer) {
            if (full) {
                *reinterpret_cast<float4 *>(a.e + i0) = make_float4(e4[0], e4[1], e4[2], e4[3]);
                if (a.m_out) *reinterpret_cast<float4 *>(a.m_out + i0) = make_float4(q4[0], q4[1], q4[2], q4[3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < t.len) {
                        a.e[i0 + q] = e4[q];
                        if (a.m_out) a.m_out[i0 + q] = q4[q];
                    }
            }
        } else if (MODE == kCompressOnly) {
            if (full) {
                *reinterpret_cast<float4 *>(a.e + i0) = make_float4(e4[0], e4[1], e4[2], e4[3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < t.len) a.e[i0 + q] = e4[q];
            }
        } else {
            float v4[4], x4[4];
            if (full) {
                const float4 vv = *reinterpret_cast<const float4 *>(a.v + i0);
                const float4 xx = *reinterpret_cast<const float4 *>(a.x + i0);
                v4[0] = vv.x; v4[1] = vv.y; v4[2] = vv.z; v4[3] = vv.w;
                x4[0] = xx.x; x4[1] = xx.y; x4[2] = xx.z; x4[3] = xx.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4[q] = (k0 + q < t.len) ? a.v[i0 + q] : 1.0f;
                    x4[q] = (k0 + q < t.len) ? a.x[i0 + q] : 0.0f;
                }
            }
            float xn[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float upd = q4[q] / (sqrtf(v4[q]) + a.eps) + a.wd * x4[q];
                xn[q] = x4[q] - a.lr * upd;
            }
            if (full) {
                *reinterpret_cast<float4 *>(a.m + i0) = make_float4(q4[0], q4[1], q4[2], q4[3]);
                *reinterpret_cast<float4 *>(a.e + i0) = make_float4(e4[0], e4[1], e4[2], e4[3]);
                *reinterpret_cast<float4 *>(a.x + i0) = make_float4(xn[0], xn[1], xn[2], xn[3]);
                if (XB) {
                    uint2 pk;
                    pk.x = float_to_bf16_bits(xn[0]) | (float_to_bf16_bits(xn[1]) << 16);
                    pk.y = float_to_bf16_bits(xn[2]) | (float_to_bf16_bits(xn[3]) << 16);
                    *reinterpret_cast<uint2 *>(a.xb + i0) = pk;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < t.len) {
                        a.m[i0 + q] = q4[q];
                        a.e[i0 + q] = e4[q];
                        a.x[i0 + q] = xn[q];
                        if (XB) a.xb[i0 + q] = (uint16_t)float_to_bf16_bits(xn[q]);
                    }
            }
        }
    }
}

__device__ __forceinline__ void load_worker_scales(const CompressArgs &a, int chunk, double *s_wscale) {
    for (int w = threadIdx.x; w < a.W; w += kBlock) s_wscale[w] = (double)a.wscales[(int64_t)w * a.n_chunks + chunk];
    __syncthreads();
}

// Pass-1 stores c where e was (e is fully rewritten by pass 2).
__device__ __forceinline__ void tile_store_c(const CompressArgs &a, const TileDesc &t, const float (&c)[kPerThread]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const int k0 = 4 * (tid + kBlock * r);
        const int64_t i0 = t.start + k0;
        if (a.aligned && k0 + 3 < t.len) {
            *reinterpret_cast<float4 *>(a.e + i0) = make_float4(c[4 * r], c[4 * r + 1], c[4 * r + 2], c[4 * r + 3]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (k0 + q < t.len) a.e[i0 + q] = c[4 * r + q];
        }
    }
}

__device__ __forceinline__ void tile_load_c(const CompressArgs &a, const TileDesc &t, float (&c)[kPerThread]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const int k0 = 4 * (tid + kBlock * r);
        const int64_t i0 = t.start + k0;
        if (a.aligned && k0 + 3 < t.len) {
            const float4 cc = *reinterpret_cast<const float4 *>(a.e + i0);
            c[4 * r] = cc.x; c[4 * r + 1] = cc.y; c[4 * r + 2] = cc.z; c[4 * r + 3] = cc.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) c[4 * r + q] = (k0 + q < t.len) ? a.e[i0 + q] : 0.0f;
        }
    }
}

constexpr int kMaxW = 1024;

// ------------------------------------------------------------- kernels
// One pass, persistent and cooperative: every workgroup of the grid is resident,
// so a tile may wait for the other tiles of its chunk.  Workgroup b takes list
// positions b, b+G, b+2G, ...; a chunk spans at most G consecutive positions, so
// its tiles sit in distinct workgroups and every wait ends.
template <int MODE, bool GBF16, bool XB>
__global__ __launch_bounds__(kBlock, 4) void k_compress_onepass(CompressArgs a) {
    __shared__ DD s_red[kWaves];
    __shared__ float s_scale;
    __shared__ uint32_t s_flag[2];
    __shared__ double s_wscale[MODE == kServer ? kMaxW : 1];
    for (int p = blockIdx.x; p < a.list_len; p += gridDim.x) {
        const int tile_id = a.list[p];
        const TileDesc t = a.tiles[tile_id];
        if (MODE == kServer) load_worker_scales(a, t.chunk, s_wscale);
        float c[kPerThread];
        tile_compute_c<MODE, GBF16>(a, t, c, s_wscale);
        tile_store_bits(a, t, c);
        const double part = tile_sum_squares(c, s_red);
        const float scale = arrive<true>(a, tile_id, t.chunk, part, s_red, &s_scale, s_flag);
        tile_finish<MODE, XB>(a, t, c, scale);
    }
}

template <int MODE, bool GBF16>
__global__ __launch_bounds__(kBlock) void k_compress_pass1(CompressArgs a) {
    __shared__ DD s_red[kWaves];
    __shared__ float s_scale;
    __shared__ uint32_t s_flag[2];
    __shared__ double s_wscale[MODE == kServer ? kMaxW : 1];
    const int tile_id = a.list[blockIdx.x];
    const TileDesc t = a.tiles[tile_id];
    if (MODE == kServer) load_worker_scales(a, t.chunk, s_wscale);
    float c[kPerThread];
    tile_compute_c<MODE, GBF16>(a, t, c, s_wscale);
    tile_store_bits(a, t, c);
    tile_store_c(a, t, c);
    const double part = tile_sum_squares(c, s_red);
    arrive<false>(a, tile_id, t.chunk, part, s_red, &s_scale, s_flag);
}

template <int MODE, bool XB>
__global__ __launch_bounds__(kBlock) void k_compress_pass2(CompressArgs a) {
    const int tile_id = a.list[blockIdx.x];
    const TileDesc t = a.tiles[tile_id];
    const float scale = a.scales[t.chunk];
    float c[kPerThread];
    tile_load_c(a, t, c);
    tile_finish<MODE, XB>(a, t, c, scale);
}

// ---------------------------------------------------------- host side
template <int MODE, bool GBF16, bool XB>
static onebit_status_t launch(const onebit_plan_s *p, CompressArgs a, hipStream_t stream) {
    const int base = MODE == kServer ? kProfServerPass1 : kProfPass1;
    // two-pass chunks first: pass 1 ...
    if (p->n_big > 0) {
        a.list = p->d_big_list;
        a.list_len = p->n_big;
        prof_before(base + 0, stream);
        hipLaunchKernelGGL((k_compress_pass1<MODE, GBF16>), dim3(p->n_big), dim3(kBlock), 0, stream, a);
        prof_after(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    if (p->n_coop > 0) {
        a.list = p->d_coop_list;
        a.list_len = p->n_coop;
        const int grid = p->n_coop < p->coop_capacity ? p->n_coop : p->coop_capacity;
        void *args[] = {&a};
        prof_before(base + 1, stream);
        hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&k_compress_onepass<MODE, GBF16, XB>),
                                                  dim3(grid), dim3(kBlock), args, 0, stream);
        prof_after(stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return hip_status(e);
        }
    }
    // ... and pass 2 once every pass-1 scale is known.
    if (p->n_big > 0) {
        a.list = p->d_big_list;
        a.list_len = p->n_big;
        prof_before(base + 2, stream);
        hipLaunchKernelGGL((k_compress_pass2<MODE, XB>), dim3(p->n_big), dim3(kBlock), 0, stream, a);
        prof_after(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    return ONEBIT_OK;
}

static int occupancy_of(const void *fn) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kBlock, 0) != hipSuccess) return 0;
    return blocks;
}

int32_t coop_capacity(int device) {
    static int32_t cached[64] = {0};
    if (device >= 0 && device < 64 && cached[device] > 0) return cached[device];
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
    if (!prop.cooperativeLaunch) return 0;
    const void *fns[] = {
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, false, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, false, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, true, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, true, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressOnly, false, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressOnly, true, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kServer, false, false>),
    };
    int per_cu = 1 << 30;
    for (const void *f : fns) {
        const int b = occupancy_of(f);
        per_cu = b < per_cu ? b : per_cu;
    }
    const int32_t cap = per_cu > 0 ? per_cu * prop.multiProcessorCount : 0;
    if (device >= 0 && device < 64) cached[device] = cap;
    return cap;
}

}  // namespace onebit

using namespace onebit;

extern "C" onebit_status_t onebit_compress_update(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                                  float *m, float *e, const float *v, float *x,
                                                  uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                                  double beta1, double eps, double weight_decay,
                                                  void *workspace, void *stream) {
    if (!plan) return ONEBIT_ERR_INVALID;
    if (g_dtype != ONEBIT_F32 && g_dtype != ONEBIT_BF16) return ONEBIT_ERR_INVALID;
    const bool update = (v != nullptr) || (x != nullptr);
    if (update && (!v || !x)) return ONEBIT_ERR_INVALID;
    if (!update && x_bf16) return ONEBIT_ERR_INVALID;
    if (plan->n_chunks == 0) return ONEBIT_OK;
    if (!scales || !workspace) return ONEBIT_ERR_INVALID;
    if (plan->n > 0 && (!g || !m || !e || !bits)) return ONEBIT_ERR_INVALID;
    const void *vec[] = {g, m, e, v, x, x_bf16};
    for (const void *q : vec)
        if (q && !aligned16(q)) return ONEBIT_ERR_ALIGN;
    if (!aligned_to(bits, 4) || !aligned_to(scales, 4) || !aligned_to(workspace, 8)) return ONEBIT_ERR_ALIGN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;

    CompressArgs a{};
    a.tiles = plan->d_tiles;
    a.chunks = plan->d_chunks;
    a.mask_iv = plan->d_mask_iv;
    a.aligned = plan->aligned ? 1 : 0;
    a.g = g;
    a.m = m;
    a.e = e;
    a.v = v;
    a.x = x;
    a.xb = x_bf16;
    a.bits = bits;
    a.scales = scales;
    a.b1 = (float)beta1;
    a.ob1 = (float)(1.0 - beta1);
    a.lr = (float)lr;
    a.eps = (float)eps;
    a.wd = (float)weight_decay;
    const WorkspaceView ws = workspace_view(workspace, plan->n_chunks);
    a.err = ws.err;
    a.chunk_words = ws.chunk_words;
    a.slots = ws.slots;
    a.spin_limit = kSpinLimit;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = g_dtype == ONEBIT_BF16;
    if (!update) return bf ? launch<kCompressOnly, true, false>(plan, a, s) : launch<kCompressOnly, false, false>(plan, a, s);
    if (x_bf16) return bf ? launch<kUpdate, true, true>(plan, a, s) : launch<kUpdate, false, true>(plan, a, s);
    return bf ? launch<kUpdate, true, false>(plan, a, s) : launch<kUpdate, false, false>(plan, a, s);
}

extern "C" onebit_status_t onebit_server_reduce(onebit_plan_t plan, int W, const uint32_t *worker_bits,
                                                const float *worker_scales, float *server_error,
                                                uint32_t *server_bits, float *server_scales, float *m_out,
                                                void *workspace, void *stream) {
    if (!plan || W < 1 || W > kMaxW) return ONEBIT_ERR_INVALID;
    if (plan->n_chunks == 0) return ONEBIT_OK;
    if (!worker_scales || !server_scales || !workspace) return ONEBIT_ERR_INVALID;
    if (plan->n > 0 && (!worker_bits || !server_error || !server_bits)) return ONEBIT_ERR_INVALID;
    if ((server_error && !aligned16(server_error)) || (m_out && !aligned16(m_out))) return ONEBIT_ERR_ALIGN;
    const void *words[] = {worker_bits, worker_scales, server_bits, server_scales};
    for (const void *q : words)
        if (q && !aligned_to(q, 4)) return ONEBIT_ERR_ALIGN;
    if (!aligned_to(workspace, 8)) return ONEBIT_ERR_ALIGN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;

    CompressArgs a{};
    a.tiles = plan->d_tiles;
    a.chunks = plan->d_chunks;
    a.mask_iv = plan->d_mask_iv;
    a.aligned = plan->aligned ? 1 : 0;
    a.e = server_error;
    a.wbits = worker_bits;
    a.wscales = worker_scales;
    a.W = W;
    a.plan_words = plan->words;
    a.n_chunks = plan->n_chunks;
    a.m_out = m_out;
    a.bits = server_bits;
    a.scales = server_scales;
    const WorkspaceView ws = workspace_view(workspace, plan->n_chunks);
    a.err = ws.err;
    a.chunk_words = ws.chunk_words;
    a.slots = ws.slots;
    a.spin_limit = kSpinLimit;
    return launch<kServer, false, false>(plan, a, static_cast<hipStream_t>(stream));
}

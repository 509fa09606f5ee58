// plan.hip -- plan construction (chunk, tile and mask tables), workspace layout,
// argument helpers and status strings.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "device_common.h"
#include "internal.h"

namespace onebit {

size_t workspace_bytes_for(int64_t n_chunks, int64_t n_tiles) {
    const size_t words = 1 + (size_t)n_chunks + (size_t)n_tiles;
    return (words * 8 + 255) / 256 * 256;
}

WorkspaceView workspace_view(void *ws, int64_t n_chunks) {
    uint64_t *w = static_cast<uint64_t *>(ws);
    return WorkspaceView{w, w + 1, w + 1 + n_chunks};
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

onebit_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return ONEBIT_OK;
    if (e == hipErrorOutOfMemory) return ONEBIT_ERR_NOMEM;
    return ONEBIT_ERR_HIP;
}

static bool offsets_ok(const int64_t *off, int64_t count) {
    if (!off || count < 0 || off[0] != 0) return false;
    for (int64_t j = 0; j < count; ++j)
        if (off[j + 1] < off[j]) return false;
    return true;
}

template <typename T>
static hipError_t upload(T **dst, const std::vector<T> &src) {
    *dst = nullptr;
    if (src.empty()) return hipSuccess;
    hipError_t e = hipMalloc(reinterpret_cast<void **>(dst), src.size() * sizeof(T));
    if (e != hipSuccess) return e;
    return hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

// ------------------------------------------------------------ profiling
struct ProfRec {
    int cls;
    hipEvent_t a, b;
};
static struct {
    bool on = false;
    uint32_t mask = 0;        // classes bracketed by events
    bool open = false;        // the last prof_before pushed a record
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
} g_prof;

static hipEvent_t prof_event() {
    if (g_prof.used == g_prof.pool.size()) {
        hipEvent_t ev = nullptr;
        if (hipEventCreate(&ev) != hipSuccess) return nullptr;
        g_prof.pool.push_back(ev);
    }
    return g_prof.pool[g_prof.used++];
}

void prof_before(int cls, hipStream_t s) {
    g_prof.open = false;
    if (!g_prof.on || !(g_prof.mask >> cls & 1u)) return;
    ProfRec r{cls, prof_event(), prof_event()};
    if (!r.a || !r.b) return;
    (void)hipEventRecord(r.a, s);
    g_prof.recs.push_back(r);
    g_prof.open = true;
}

void prof_after(hipStream_t s) {
    if (!g_prof.open) return;
    g_prof.open = false;
    (void)hipEventRecord(g_prof.recs.back().b, s);
}

__global__ void k_fill_zero(uint64_t *p, int64_t words) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace onebit

using namespace onebit;

extern "C" const char *onebit_status_string(onebit_status_t s) {
    switch (s) {
        case ONEBIT_OK: return "ok";
        case ONEBIT_ERR_INVALID: return "invalid argument";
        case ONEBIT_ERR_ALIGN: return "misaligned pointer";
        case ONEBIT_ERR_HIP: return "HIP runtime error";
        case ONEBIT_ERR_NOMEM: return "out of device memory";
        case ONEBIT_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

extern "C" void onebit_plan_destroy(onebit_plan_t p) {
    if (!p) return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(p->device);
    (void)hipFree(p->d_tiles);
    (void)hipFree(p->d_chunks);
    (void)hipFree(p->d_mask_iv);
    (void)hipFree(p->d_onepass_list);
    (void)hipFree(p->d_big_list);
    (void)hipFree(p->d_big_chunks);
    if (prev >= 0) (void)hipSetDevice(prev);
    delete p;
}

namespace onebit {

// Host tables of a plan: merged masked intervals, per-chunk and per-tile
// descriptors.  Pure host code (no device is touched).
struct HostTables {
    std::vector<int64_t> iv;  // [a, b) pairs of masked elements, sorted, disjoint, non-adjacent
    std::vector<TileDesc> tiles;
    std::vector<ChunkDesc> chunks;
    int64_t n = 0;
    int64_t words = 0;
    int32_t max_chunk_tiles = 0;
    bool aligned = true;
};

static onebit_status_t build_tables(const int64_t *chunk_offsets, int64_t n_chunks, const int64_t *tensor_offsets,
                                    const uint8_t *tensor_keep, int64_t n_tensors, HostTables &T) {
    if (!offsets_ok(chunk_offsets, n_chunks)) return ONEBIT_ERR_INVALID;
    const int64_t n = chunk_offsets[n_chunks];
    if (tensor_offsets) {
        if (!offsets_ok(tensor_offsets, n_tensors) || tensor_offsets[n_tensors] != n) return ONEBIT_ERR_INVALID;
    } else if (tensor_keep) {
        return ONEBIT_ERR_INVALID;
    }
    if (n_chunks > (1ll << 30)) return ONEBIT_ERR_UNSUPPORTED;
    T.n = n;

    // masked intervals: runs of consecutive masked, non-empty tensors
    if (tensor_offsets && tensor_keep) {
        for (int64_t t = 0; t < n_tensors; ++t) {
            const int64_t a = tensor_offsets[t], b = tensor_offsets[t + 1];
            if (tensor_keep[t] || a == b) continue;
            if (!T.iv.empty() && T.iv.back() == a)
                T.iv.back() = b;
            else {
                T.iv.push_back(a);
                T.iv.push_back(b);
            }
        }
    }
    const size_t n_iv = T.iv.size() / 2;

    T.chunks.resize((size_t)n_chunks);
    int64_t word = 0;
    size_t ivp = 0;  // first interval that may still touch the current tile
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t o = chunk_offsets[j], len = chunk_offsets[j + 1] - o;
        if (o % 4 != 0) T.aligned = false;
        const int64_t nt = len > 0 ? (len + kTile - 1) / kTile : 1;
        if ((int64_t)T.tiles.size() + nt > (1ll << 31) - 1) return ONEBIT_ERR_UNSUPPORTED;
        T.chunks[j] = ChunkDesc{len, (int32_t)T.tiles.size(), (int32_t)nt};
        if (nt > T.max_chunk_tiles) T.max_chunk_tiles = (int32_t)nt;
        for (int64_t k = 0; k < nt; ++k) {
            TileDesc t{};
            t.start = o + k * kTile;
            t.len = (int32_t)std::max<int64_t>(0, std::min<int64_t>(kTile, len - k * kTile));
            t.word = word + k * (kTile / 32);
            t.chunk = (int32_t)j;
            const int64_t lo = t.start, hi = t.start + t.len;
            while (ivp < n_iv && T.iv[2 * ivp + 1] <= lo) ++ivp;
            size_t q = ivp;
            while (q < n_iv && T.iv[2 * q] < hi) ++q;
            t.mask_lo = (int32_t)ivp;
            t.mask_hi = (int32_t)q;
            if (t.len == 0) {
                t.mask_lo = t.mask_hi = 0;
            } else if (q == ivp + 1 && T.iv[2 * ivp] <= lo && T.iv[2 * ivp + 1] >= hi) {
                t.mask_lo = -1;  // one interval covers the whole tile
                t.mask_hi = 0;
            }
            T.tiles.push_back(t);
        }
        word += (len + 31) / 32;
    }
    T.words = word;
    return ONEBIT_OK;
}

}  // namespace onebit

extern "C" onebit_status_t onebit_plan_host_tables(const int64_t *chunk_offsets, int64_t n_chunks,
                                                   const int64_t *tensor_offsets, const uint8_t *tensor_keep,
                                                   int64_t n_tensors, int64_t *n_tiles, int64_t *n_words,
                                                   int64_t *out_tiles, int64_t *n_mask_iv, int64_t *out_mask_iv) {
    HostTables T;
    const onebit_status_t st = build_tables(chunk_offsets, n_chunks, tensor_offsets, tensor_keep, n_tensors, T);
    if (st != ONEBIT_OK) return st;
    if (n_tiles) *n_tiles = (int64_t)T.tiles.size();
    if (n_words) *n_words = T.words;
    if (n_mask_iv) *n_mask_iv = (int64_t)T.iv.size() / 2;
    if (out_tiles) {
        for (size_t i = 0; i < T.tiles.size(); ++i) {
            const TileDesc &t = T.tiles[i];
            int64_t *r = out_tiles + 6 * i;
            r[0] = t.start;
            r[1] = t.word;
            r[2] = t.len;
            r[3] = t.chunk;
            r[4] = t.mask_lo;
            r[5] = t.mask_hi;
        }
    }
    if (out_mask_iv)
        for (size_t i = 0; i < T.iv.size(); ++i) out_mask_iv[i] = T.iv[i];
    return ONEBIT_OK;
}

extern "C" onebit_status_t onebit_plan_create(const int64_t *chunk_offsets, int64_t n_chunks,
                                              const int64_t *tensor_offsets, const uint8_t *tensor_keep,
                                              int64_t n_tensors, onebit_plan_t *out) {
    if (!out) return ONEBIT_ERR_INVALID;
    *out = nullptr;
    HostTables T;
    const onebit_status_t st = build_tables(chunk_offsets, n_chunks, tensor_offsets, tensor_keep, n_tensors, T);
    if (st != ONEBIT_OK) return st;

    onebit_plan_s *p = new (std::nothrow) onebit_plan_s();
    if (!p) return ONEBIT_ERR_NOMEM;
    if (hipGetDevice(&p->device) != hipSuccess) {
        delete p;
        return ONEBIT_ERR_HIP;
    }
    p->n = T.n;
    p->n_chunks = n_chunks;
    p->n_mask_iv = (int64_t)T.iv.size() / 2;
    p->n_tiles = (int64_t)T.tiles.size();
    p->words = T.words;
    p->aligned = T.aligned;
    p->max_chunk_tiles = T.max_chunk_tiles;

    // one-pass chunks (at most onepass_depth() times the resident workgroups: the
    // one-pass kernel keeps that many tiles in flight per workgroup) and two-pass
    // chunks
    p->resident_capacity = resident_capacity(p->device);
    std::vector<int32_t> onepass, big, big_chunks;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const ChunkDesc &c = T.chunks[j];
        const bool one_pass = (int64_t)c.ntiles <= (int64_t)onepass_depth() * (int64_t)p->resident_capacity;
        std::vector<int32_t> &dst = one_pass ? onepass : big;
        for (int32_t k = 0; k < c.ntiles; ++k) dst.push_back(c.first_tile + k);
        if (!one_pass) big_chunks.push_back((int32_t)j);
        if (one_pass && c.ntiles > p->max_onepass_chunk_tiles) p->max_onepass_chunk_tiles = c.ntiles;
    }
    p->n_onepass = (int32_t)onepass.size();
    p->n_big = (int32_t)big.size();
    p->n_big_chunks = (int32_t)big_chunks.size();

    hipError_t e = upload(&p->d_tiles, T.tiles);
    if (e == hipSuccess) e = upload(&p->d_chunks, T.chunks);
    if (e == hipSuccess) e = upload(&p->d_mask_iv, T.iv);
    if (e == hipSuccess) e = upload(&p->d_onepass_list, onepass);
    if (e == hipSuccess) e = upload(&p->d_big_list, big);
    if (e == hipSuccess) e = upload(&p->d_big_chunks, big_chunks);
    if (e != hipSuccess) {
        onebit_plan_destroy(p);
        return hip_status(e);
    }
    *out = p;
    return ONEBIT_OK;
}

extern "C" int64_t onebit_plan_elements(onebit_plan_t p) { return p ? p->n : -1; }
extern "C" int64_t onebit_plan_chunks(onebit_plan_t p) { return p ? p->n_chunks : -1; }
extern "C" int64_t onebit_plan_words(onebit_plan_t p) { return p ? p->words : -1; }

extern "C" size_t onebit_plan_workspace_bytes(onebit_plan_t p) {
    return p ? workspace_bytes_for(p->n_chunks, p->n_tiles) : 0;
}

extern "C" onebit_status_t onebit_workspace_init(void *workspace, size_t bytes, void *stream) {
    if (!workspace || bytes % 8 != 0) return ONEBIT_ERR_INVALID;
    if (!aligned_to(workspace, 8)) return ONEBIT_ERR_ALIGN;
    const int64_t words = (int64_t)(bytes / 8);
    if (words == 0) return ONEBIT_OK;
    const int64_t blocks = std::min<int64_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint64_t *>(workspace), words);
    return hip_status(hipGetLastError());
}

extern "C" onebit_status_t onebit_workspace_status(const void *workspace, uint64_t *out, void *stream) {
    if (!workspace || !out) return ONEBIT_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(out, workspace, sizeof(uint64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return hip_status(e);
}

extern "C" void onebit_profile_begin_classes(uint32_t class_mask) {
    g_prof.on = true;
    g_prof.mask = class_mask;
    g_prof.open = false;
    g_prof.recs.clear();
    g_prof.used = 0;
}

extern "C" void onebit_profile_begin(void) { onebit_profile_begin_classes((1u << kProfClasses) - 1u); }

extern "C" onebit_status_t onebit_profile_end(double *total_ms, int64_t *launches) {
    g_prof.on = false;
    onebit_status_t st = ONEBIT_OK;
    for (int c = 0; c < kProfClasses; ++c) {
        if (total_ms) total_ms[c] = 0.0;
        if (launches) launches[c] = 0;
    }
    for (const ProfRec &r : g_prof.recs) {
        if (hipEventSynchronize(r.b) != hipSuccess) {
            st = ONEBIT_ERR_HIP;
            continue;
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            st = ONEBIT_ERR_HIP;
            continue;
        }
        if (total_ms) total_ms[r.cls] += ms;
        if (launches) launches[r.cls] += 1;
    }
    g_prof.recs.clear();
    g_prof.used = 0;
    return st;
}

extern "C" int32_t onebit_device_resident_capacity(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    return resident_capacity(dev);
}

extern "C" int64_t onebit_onepass_max_elements(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    return (int64_t)onepass_depth() * (int64_t)resident_capacity(dev) * (int64_t)kTile;
}

extern "C" void onebit_plan_stats(onebit_plan_t p, int64_t *out6) {
    if (!p || !out6) return;
    out6[0] = p->n_tiles;
    out6[1] = p->n_onepass;
    out6[2] = p->n_big;
    out6[3] = p->resident_capacity;
    out6[4] = p->max_chunk_tiles;
    out6[5] = p->aligned ? 1 : 0;
}

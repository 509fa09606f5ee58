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
// How: the flat vector is cut into tiles of 2048 elements (256 threads x 8).
// A tile computes its c, writes its sign words, and posts its fp64 partial sum
// of squares.  The chunk scale needs every tile of the chunk, so
//  - chunks of at most 3R tiles (R = co-resident workgroups) are done in ONE pass
//    by a persistent kernel whose grid is at most R workgroups, so that every
//    workgroup is resident: each tile parks c in LDS, waits for its chunk's scale
//    while the next tiles stream, then finishes -- HBM sees each input once and
//    each output once;
//  - larger chunks take two passes: pass 1 stores c in place of e, pass 2 reads it
//    back with v and x once the chunk scale is known.
// Cross-workgroup communication uses only single-location relaxed agent-scope
// atomics on self-validating words (a tagged partial per tile, an {epoch, scale}
// word per chunk); no cache-wide write-back or invalidate is ever needed, and a
// zeroed workspace is always ready for the next call.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace onebit {

// kUpdatePM / kCompressPM: the update / compress-only modes with the momentum held
// in its compressed form (the previous step's sign words and chunk scales) instead
// of an fp32 array.
// kServerWide: the server stage for more than kWBatch workers (its exact-sum tables
// are built batch by batch; a separate instantiation, so that the common case of at
// most kWBatch workers keeps its own code).
enum Mode { kUpdate = 0, kCompressOnly = 1, kServer = 2, kUpdatePM = 3, kCompressPM = 4, kServerWide = 5 };
constexpr bool is_server(int mode) { return mode == kServer || mode == kServerWide; }
constexpr bool packed_m(int mode) { return mode == kUpdatePM || mode == kCompressPM; }
constexpr bool compress_only(int mode) { return mode == kCompressOnly || mode == kCompressPM; }

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
    const uint32_t *m_bits;  // packed modes: m = decompression of these words and scales,
    const float *m_scales;   // zero where m_mask (uint8 per element, nullable) is 0
    const uint8_t *m_mask;
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
    double w_pow2_scale;  // 1/W when W is a power of two, else 0
    float *m_out;
    // outputs
    uint32_t *bits;
    float *scales;
    // hyperparameters (binary32)
    float b1, ob1, lr, eps, wd;
    // workspace
    uint64_t *err;
    uint64_t *publish;
    uint64_t *slots;
    uint32_t spin_limit;
};

// Bound of every cross-workgroup wait (iterations of a short sleep and a reload).
// A wait that runs out records an error in the workspace; from then on no wait
// of any workgroup spins again, so a kernel always drains in bounded time.
constexpr uint32_t kSpinLimit = 1u << 20;
// Limit used by the next launches (diagnostics can lower it to exercise the
// failure path; a wait that gives up records an error in the workspace).  Atomic:
// any host thread may set it while others launch.
static std::atomic<uint32_t> g_spin_limit{kSpinLimit};
// Diagnostic cap on the one-pass grid (0 = none): lets the tests run the chunk-norm
// exchange with fewer resident workgroups than the device holds.
static std::atomic<int32_t> g_grid_cap{0};

__device__ __forceinline__ bool give_up(const CompressArgs &a, uint32_t spins) {
    return spins >= a.spin_limit || ((spins & 255u) == 255u && ld_agent(a.err) != 0);
}

// ---------------------------------------------------------------- tile: c
// Thread t of a tile owns elements 4(t + 256 r) .. +3, r < kGroups: every load
// instruction of a workgroup covers 4 KiB of consecutive fp32.  Addresses are a
// uniform per-tile base plus a 32-bit lane offset.  A tile is "full" when it
// holds kTile elements and starts on a multiple of 4 (the common case); other
// tiles take per-element guarded accesses.
__device__ __forceinline__ bool tile_full(const CompressArgs &a, const TileDesc &t) {
    return a.aligned && t.len == kTile;
}
__device__ __forceinline__ uint32_t lane_k0(int r) { return 4u * (threadIdx.x + kBlock * r); }

template <int GT>
__device__ __forceinline__ void load_g4(const void *g, int64_t start, uint32_t k0, float (&g4)[4]) {
    if (GT != kGradF32) {
        const uint2 h = ld_stream(reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(g) + start + k0));
        g4[0] = half_bits_to_float<GT>(h.x & 0xffffu);
        g4[1] = half_bits_to_float<GT>(h.x >> 16);
        g4[2] = half_bits_to_float<GT>(h.y & 0xffffu);
        g4[3] = half_bits_to_float<GT>(h.y >> 16);
    } else {
        const float4 h = ld_stream(reinterpret_cast<const float4 *>(static_cast<const float *>(g) + start + k0));
        g4[0] = h.x; g4[1] = h.y; g4[2] = h.z; g4[3] = h.w;
    }
}

__device__ __forceinline__ void load4(const float *base, uint32_t k0, float (&v)[4]) {
    const float4 h = ld_stream(reinterpret_cast<const float4 *>(base + k0));
    v[0] = h.x; v[1] = h.y; v[2] = h.z; v[3] = h.w;
}

// Server tiles: average of the W workers' decompressed values, summed in fp64 in
// worker order 0..W-1.  Workers are taken kWBatch at a time: their scales for the
// chunk and the tile's packed words are staged in LDS (each worker's words load as
// one 256-byte run), then every thread adds +-s for its elements as fma(+-1, s,
// acc), the +-1.0 built from the sign bit in two instructions (server 0.304 ->
// 0.294 ms on 16 x 64M against a sign-bit xor on s).  The server error is loaded
// before the words are staged, so the two loads are in flight together (0.291 ->
// 0.285 ms).  For scales whose partial sums are all exact, the sums come from
// per-group tables instead (below; W = 16: 0.284 -> 0.253 ms; with more than
// kWBatch workers the kServerWide instantiation builds them batch by batch).
constexpr int kWBatch = 16;
constexpr int kTileWords = kTile / 32;

// Exact-sum tables: for each group of four workers of a batch, the 16 signed sums
// +-s_4g +-s_4g+1 +-s_4g+2 +-s_4g+3 (bit k of the entry index set: worker 4g+k
// negative), so that an element adds four table entries per batch of kWBatch
// workers instead of kWBatch scales.  The
// regrouped sum equals the ordered one exactly when no partial sum of either rounds:
// every scale is finite and, with u the smallest unit in the last place of the
// nonzero scales (2^(e_min - 150) for biased exponent fields e, subnormals counted
// as e = 1), every partial sum is an integer multiple of u below W * 2^(e_max - 126)
// <= 2^53 u, i.e. e_max - e_min <= 29 - ceil(log2 W).  Both forms start from +0 and
// never produce -0, so zeros agree in sign too.  Otherwise the ordered loop runs.
constexpr int kWGroups = kWBatch / 4;
constexpr int kServerLdsDoubles = kWBatch + kWGroups * 16 + 1;  // scales, tables, exact flag

// Bit q of a 4-bit value moved to bit 8q (the four copies of the product do not
// overlap, so no carry crosses them).
__device__ __forceinline__ uint32_t spread_nibble(uint32_t n) { return (n * 0x00204081u) & 0x01010101u; }

template <bool WIDE>
__device__ __forceinline__ void server_tile_c(const CompressArgs &a, const TileDesc &t, float (&c)[kPerThread],
                                              double *s_wscale_d, uint32_t *s_words) {
    const bool full = tile_full(a, t);
    const int nwords = (t.len + 31) / 32;
    const float *eb = a.e + t.start;
    float es[kPerThread];
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        float e4[4];
        if (full) {
            load4(eb, k0, e4);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) e4[q] = (k0 + q < (uint32_t)t.len) ? eb[k0 + q] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) es[4 * r + q] = e4[q];
    }
    double acc[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) acc[j] = 0.0;
    for (int w0 = 0; w0 < a.W; w0 += kWBatch) {
        const int wn = min(kWBatch, a.W - w0);
        __syncthreads();  // previous batch fully consumed
        double *s_tab = s_wscale_d + kWBatch;
        int *s_exact = reinterpret_cast<int *>(s_wscale_d + kWBatch + kWGroups * 16);
        const bool tables = WIDE || a.W <= kWBatch;
        const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        if (tables && wave == 0) {
            // wave 0: this batch's scales and tables, and (with the first batch)
            // whether the regrouped sum is exact over all W workers.  The lane index
            // is made opaque here so that nothing derived from it is hoisted out of
            // the tile loop and held in registers for the whole kernel.
            int j = (int)threadIdx.x;
            asm volatile("" : "+v"(j));
            const int wj = WIDE ? w0 + j : j;  // one batch only when !WIDE
            const float sv = j < wn ? a.wscales[(int64_t)wj * a.n_chunks + t.chunk] : 0.0f;
            if (j < wn) s_wscale_d[j] = (double)sv;
            if (!WIDE || w0 == 0) {
                // lane j: worker j's scale (in sv), then with WIDE workers j + 64,
                // j + 128, ... (from j itself for the lanes past the first batch)
                const uint32_t bits = __float_as_uint(sv) & 0x7FFFFFFFu;
                const int ef = (int)(bits >> 23);
                int emin = bits != 0u ? max(ef, 1) : 255, emax = bits != 0u ? max(ef, 1) : 0;
                int bad = ef == 255;
                if (WIDE) {
                    for (int w = j < kWBatch ? j + 64 : j; w < a.W; w += 64) {
                        const uint32_t wb = __float_as_uint(a.wscales[(int64_t)w * a.n_chunks + t.chunk]) & 0x7FFFFFFFu;
                        const int we = (int)(wb >> 23);
                        if (wb != 0u) {
                            emin = min(emin, max(we, 1));
                            emax = max(emax, max(we, 1));
                        }
                        bad |= we == 255;
                    }
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    emin = min(emin, __shfl_xor(emin, o));
                    emax = max(emax, __shfl_xor(emax, o));
                    bad |= __shfl_xor(bad, o);
                }
                const int lg = 32 - __clz((WIDE ? a.W : wn) - 1);  // ceil(log2 W), 0 for W = 1
                if (j == 0) *s_exact = !bad && (emax == 0 || emax - emin <= 29 - lg);
            }
            // table entry j (lane j) of group j / 16 from the scales of lanes 4g .. 4g+3
            const int g = j >> 4;
            double T = 0.0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float sw = __shfl(sv, 4 * g + k);
                if (4 * g + k < wn) T = __fma_rn((j >> k) & 1 ? -1.0 : 1.0, (double)sw, T);
            }
            s_tab[j] = T;
        } else if (!tables) {
            for (int w = threadIdx.x; w < wn; w += kBlock)
                s_wscale_d[w] = (double)a.wscales[(int64_t)(w0 + w) * a.n_chunks + t.chunk];
        }
        // a full batch of a full tile with 16-byte aligned rows: one 16-byte load per
        // thread (thread k takes words 4k..4k+3 of the batch), else one word each
        const bool vec = kWBatch * kTileWords == 4 * kBlock && full && wn == kWBatch &&
                         (((uintptr_t)a.wbits | (uintptr_t)a.plan_words * 4u | (uintptr_t)t.word * 4u) & 15u) == 0;
        if (vec) {
            const int w = threadIdx.x / (kTileWords / 4), i = 4 * (threadIdx.x % (kTileWords / 4));
            reinterpret_cast<uint4 *>(s_words)[threadIdx.x] =
                *reinterpret_cast<const uint4 *>(a.wbits + (int64_t)(w0 + w) * a.plan_words + t.word + i);
        } else {
            for (int k = threadIdx.x; k < wn * kTileWords; k += kBlock) {
                const int w = k / kTileWords, i = k % kTileWords;
                s_words[k] = i < nwords ? a.wbits[(int64_t)(w0 + w) * a.plan_words + t.word + i] : 0u;
            }
        }
        __syncthreads();
        if (tables && *s_exact) {
            const int ng = (wn + 3) >> 2;
#pragma unroll
            for (int r = 0; r < kGroups; ++r) {
                const uint32_t k0 = lane_k0(r);
                const uint32_t wi = k0 >> 5;
                const uint32_t sh = k0 & 31u;
#pragma unroll 1
                for (int g = 0; g < ng; ++g) {
                    // byte q of idx: the entry index of element q (bit k from worker 4g+k)
                    uint32_t idx = 0u;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t nib = __builtin_amdgcn_ubfe(s_words[(4 * g + k) * kTileWords + wi], sh, 4);
                        idx |= spread_nibble(nib) << k;
                    }
                    const double *tg = s_tab + 16 * g;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[4 * r + q] = __dadd_rn(acc[4 * r + q], tg[__builtin_amdgcn_ubfe(idx, 8 * q, 4)]);
                }
            }
            continue;
        }
#pragma unroll
        for (int r = 0; r < kGroups; ++r) {
            const uint32_t k0 = lane_k0(r);
            const uint32_t wi = k0 >> 5;
            const uint32_t sh = k0 & 31u;
            for (int w = 0; w < wn; ++w) {
                const uint32_t word = s_words[w * kTileWords + wi];
                const double sw = s_wscale_d[w];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // +-1.0 from bit sh + q of the word: the bit shifted into the sign,
                    // 1.0's exponent field or-ed in ((a & b) | c, truth table 0xEA);
                    // fma(+-1, s, acc) = acc +- s with one rounding, as the ordered sum
                    const uint32_t hi = __builtin_amdgcn_bitop3_b32(word << (31u - sh - (uint32_t)q), 0x80000000u,
                                                                    0x3FF00000u, 0xEA);
                    acc[4 * r + q] = __fma_rn(__hiloint2double((int)hi, 0), sw, acc[4 * r + q]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // a power-of-two W divides exactly by scaling
            const double x = acc[4 * r + q];
            const double mean = a.w_pow2_scale != 0.0 ? __dmul_rn(x, a.w_pow2_scale) : __ddiv_rn(x, (double)a.W);
            c[4 * r + q] = (full || k0 + q < (uint32_t)t.len) ? add_rn((float)mean, es[4 * r + q]) : 0.0f;
        }
    }
}

// Masked elements among this thread's 2 x 4 elements of a tile: bit 4r+q for
// element lane_k0(r)+q, from one pass over the intervals that touch the tile.
__device__ __forceinline__ uint32_t thread_mask_bits(const CompressArgs &a, const TileDesc &t) {
    if (t.mask_lo < 0) return 0xFFu;
    uint32_t bits = 0u;
    for (int k = t.mask_lo; k < t.mask_hi; ++k) {
        const int64_t lo = a.mask_iv[2 * k], hi = a.mask_iv[2 * k + 1];
#pragma unroll
        for (int r = 0; r < kGroups; ++r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = t.start + (int64_t)lane_k0(r) + q;
                bits |= (uint32_t)((i >= lo) & (i < hi)) << (4 * r + q);
            }
        }
    }
    return bits;
}

// Elements of this thread whose byte in the caller's element mask is 0 (same bit
// layout as thread_mask_bits; none without a mask).
__device__ __forceinline__ uint32_t element_mask_bits(const CompressArgs &a, const TileDesc &t) {
    if (!a.m_mask) return 0u;
    uint32_t bits = 0u;
    const bool full = tile_full(a, t);
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        if (full) {  // four mask bytes as one aligned word
            const uint32_t w = *reinterpret_cast<const uint32_t *>(a.m_mask + t.start + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (((w >> (8 * q)) & 0xffu) == 0) bits |= 1u << (4 * r + q);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t k = k0 + q;
                if (k < (uint32_t)t.len && a.m_mask[t.start + k] == 0) bits |= 1u << (4 * r + q);
            }
        }
    }
    return bits;
}

// The momentum of four elements from the previous step's packed form: +-scale by
// sign bit, 0 for masked elements (as the fp32 form holds them).
__device__ __forceinline__ void load_packed_m4(const CompressArgs &a, const TileDesc &t, uint32_t k0,
                                               uint32_t masked4, uint32_t dropped4, float (&m4)[4]) {
    const float s = a.m_scales[t.chunk];
    const uint32_t wi = k0 >> 5;
    const uint32_t word = wi < (((uint32_t)t.len + 31u) >> 5) ? a.m_bits[t.word + wi] : 0u;
    const uint32_t nib = word >> (k0 & 31u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float mq = ((nib >> q) & 1u) ? -s : s;
        m4[q] = ((masked4 >> q) & 1u) ? 0.0f : (((dropped4 >> q) & 1u) ? mul_rn(mq, 0.0f) : mq);
    }
}

template <int MODE, int GT>
__device__ __forceinline__ void tile_compute_c(const CompressArgs &a, const TileDesc &t,
                                               float (&c)[kPerThread], double *s_wscale_d,
                                               uint32_t *s_words) {
    const bool full = tile_full(a, t);
    if (!is_server(MODE)) {
        const float *mb = packed_m(MODE) ? nullptr : a.m + t.start;
        const float *eb = a.e + t.start;
        // the packed momentum is 0 where the fp32 one would hold 0: +0 in masked
        // tensors in the update mode (whose step stores +0), and +-s * 0 where the
        // caller's element mask is 0 (as the finish multiplies by the mask)
        const uint32_t masked = MODE == kUpdatePM ? thread_mask_bits(a, t) : 0u;
        const uint32_t dropped = packed_m(MODE) ? element_mask_bits(a, t) : 0u;
#pragma unroll
        for (int r = 0; r < kGroups; ++r) {
            const uint32_t k0 = lane_k0(r);
            float g4[4], m4[4], e4[4];
            if (packed_m(MODE)) load_packed_m4(a, t, k0, (masked >> (4 * r)) & 0xFu, (dropped >> (4 * r)) & 0xFu, m4);
            if (full) {
                load_g4<GT>(a.g, t.start, k0, g4);
                if (!packed_m(MODE)) load4(mb, k0, m4);
                load4(eb, k0, e4);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t k = k0 + q;
                    const bool in = k < (uint32_t)t.len;
                    g4[q] = in ? (GT != kGradF32 ? half_bits_to_float<GT>(static_cast<const uint16_t *>(a.g)[t.start + k])
                                                 : static_cast<const float *>(a.g)[t.start + k])
                               : 0.0f;
                    if (!packed_m(MODE)) m4[q] = in ? mb[k] : 0.0f;
                    e4[q] = in ? eb[k] : 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float m1 = add_rn(mul_rn(a.b1, m4[q]), mul_rn(a.ob1, g4[q]));
                const float cq = add_rn(m1, e4[q]);
                c[4 * r + q] = (full || k0 + q < (uint32_t)t.len) ? cq : 0.0f;
            }
        }
    } else {
        server_tile_c<MODE == kServerWide>(a, t, c, s_wscale_d, s_words);
    }
}

// ------------------------------------------------------- tile: sign words
__device__ __forceinline__ void tile_store_bits(const CompressArgs &a, const TileDesc &t,
                                                const float (&c)[kPerThread]) {
    uint32_t *wb = a.bits + t.word;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        const uint32_t nib = (c[4 * r + 0] < 0.0f ? 1u : 0u) | (c[4 * r + 1] < 0.0f ? 2u : 0u) |
                             (c[4 * r + 2] < 0.0f ? 4u : 0u) | (c[4 * r + 3] < 0.0f ? 8u : 0u);
        const uint32_t word = or_over_8_lanes(nib << (k0 & 31u));
        if ((threadIdx.x & 7) == 0 && k0 < (uint32_t)t.len) wb[k0 >> 5] = word;
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

// Sum of a chunk's posted partials, read from its tile slots.  Each thread takes
// a fixed subset in a fixed order and the waves combine in a fixed tree, so the
// result does not depend on which tile finished last.  All loads of a batch are
// in flight before any is checked; a slot that is not yet visible is re-polled.
// Slots are cleared after reading (zero = empty for the next call).
template <int NT = kBlock, int kBatch = 8>
__device__ double chunk_sum(const CompressArgs &a, const ChunkDesc &ch, DD *s_red, double *s_total) {
    constexpr int kW = NT / 64;
    DD acc = {0.0, 0.0};
    for (int base = 0; base < ch.ntiles; base += NT * kBatch) {
        uint64_t w[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int k = base + u * NT + (int)threadIdx.x;
            w[u] = k < ch.ntiles ? ld_agent(a.slots + ch.first_tile + k) : kTag;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int k = base + u * NT + (int)threadIdx.x;
            if (k < ch.ntiles) {
                uint64_t *slot = a.slots + ch.first_tile + k;
                uint32_t spins = 0;
                while (!(w[u] & kTag) && !give_up(a, spins)) {
                    spin_pause();
                    w[u] = ld_agent(slot);
                    ++spins;
                }
                if (!(w[u] & kTag)) st_agent(a.err, 1);
                dd_add_term(acc, untag_partial(w[u]));
                st_agent(slot, 0);
            }
        }
    }
    acc = wave_sum_dd(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) s_red[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        DD t = s_red[0];
#pragma unroll
        for (int w = 1; w < kW; ++w) t = dd_add(t, s_red[w]);
        *s_total = __dadd_rn(t.hi, t.lo);
    }
    __syncthreads();
    const double total = *s_total;
    __syncthreads();
    return total;
}

__device__ __forceinline__ float scale_of(double S, int64_t len) {
    return len > 0 ? (float)__ddiv_rn(__dsqrt_rn(S), __dsqrt_rn((double)len)) : 0.0f;
}

// Slot loads in flight per thread when a tile of the one-pass kernel finalizes its
// chunk.  This path is inlined into every tile, so its registers count for the
// whole kernel: with 8 (16 VGPRs of slot words) it set the kernel's peak, and
// the update and packed-momentum variants spilled; with 4 they do not.
constexpr int kFinalizeBatch = 4;

// What a workgroup knows about a tile it has posted.
struct Posted {
    uint32_t epoch;  // publish epoch of the chunk read before posting
    uint32_t mine;   // this workgroup finalized the chunk (it holds its last tile)
    float scale;     // valid when mine
};

// Post a tile's partial: read the chunk's publish epoch (and wait for that read to
// complete, so it precedes the post), then store the tagged partial in the tile's
// own slot -- no read-modify-write, so tiles never contend for one word.  The
// workgroup holding the chunk's last tile then sums all slots and publishes
// {epoch + 1, scale}.  With at most onepass_depth() tiles of a chunk per workgroup,
// all earlier tiles of the chunk are posted by workgroups that do not wait on it.
// ch_ahead: the chunk's descriptor when the caller loaded it ahead, else null (read
// here).
template <bool FINALIZE>
__device__ Posted post_tile(const CompressArgs &a, int tile_id, int chunk, const ChunkDesc *ch_ahead, double partial,
                            DD *s_red, uint32_t *s_u32, double *s_total) {
    if (threadIdx.x == 0) {
        const uint64_t pw = ld_agent(a.publish + chunk);
        s_u32[0] = (uint32_t)(pw >> 32);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        st_agent(a.slots + tile_id, tag_partial(partial));
    }
    __syncthreads();
    Posted r{s_u32[0], 0u, 0.0f};
    __syncthreads();
    if (FINALIZE) {
        const ChunkDesc ch = ch_ahead ? *ch_ahead : a.chunks[chunk];
        if (tile_id == ch.first_tile + ch.ntiles - 1) {
            r.mine = 1u;
            r.scale = scale_of(chunk_sum<kBlock, kFinalizeBatch>(a, ch, s_red, s_total), ch.len);
            if (threadIdx.x == 0) {
                a.scales[chunk] = r.scale;
                st_agent(a.publish + chunk,
                         ((uint64_t)(uint32_t)(r.epoch + 1u) << 32) | (uint64_t)__float_as_uint(r.scale));
            }
        }
    }
    return r;
}

// Scale of a posted tile's chunk: computed here if this workgroup finalized it,
// else read from the chunk's publish word once its epoch has advanced.
__device__ float wait_scale(const CompressArgs &a, int chunk, const Posted &r, uint32_t *s_u32) {
    if (r.mine) return r.scale;
    if (threadIdx.x == 0) {
        const uint64_t *pub = a.publish + chunk;
        const uint32_t want = r.epoch + 1u;
        uint64_t w = ld_agent(pub);
        uint32_t spins = ld_agent(a.err) != 0 ? a.spin_limit : 0u;
        while ((uint32_t)(w >> 32) != want && !give_up(a, spins)) {
            spin_pause();
            w = ld_agent(pub);
            ++spins;
        }
        if ((uint32_t)(w >> 32) != want) st_agent(a.err, 2);
        s_u32[1] = (uint32_t)w;
    }
    __syncthreads();
    const float scale = __uint_as_float(s_u32[1]);
    __syncthreads();
    return scale;
}


__device__ __forceinline__ void store4(float *base, uint32_t k0, const float (&v)[4]) {
    st_stream(reinterpret_cast<float4 *>(base + k0), make_float4(v[0], v[1], v[2], v[3]));
}

// ------------------------------------------------------- tile: finish
// q = +-scale, e = c - q, masked -> 0, then the frozen-v step (update mode).
template <int MODE, bool XB>
__device__ __forceinline__ void tile_finish(const CompressArgs &a, const TileDesc &t,
                                            const float (&c)[kPerThread], float scale) {
    const bool full = tile_full(a, t);
    const uint32_t masked = !is_server(MODE) ? thread_mask_bits(a, t) : 0u;
    float *eb = a.e + t.start;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        float q4[4], e4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float cq = c[4 * r + q];
            q4[q] = cq < 0.0f ? -scale : scale;
            e4[q] = sub_rn(cq, q4[q]);
            if ((masked >> (4 * r + q)) & 1u) {
                q4[q] = 0.0f;
                e4[q] = 0.0f;
            }
        }
        if (is_server(MODE)) {
            float *mo = a.m_out ? a.m_out + t.start : nullptr;
            if (full) {
                store4(eb, k0, e4);
                if (mo) store4(mo, k0, q4);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < (uint32_t)t.len) {
                        eb[k0 + q] = e4[q];
                        if (mo) mo[k0 + q] = q4[q];
                    }
            }
        } else if (compress_only(MODE)) {
            if (full) {
                store4(eb, k0, e4);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < (uint32_t)t.len) eb[k0 + q] = e4[q];
            }
        } else {
            const float *vb = a.v + t.start;
            float *xb = a.x + t.start;
            float *mb = MODE == kUpdatePM ? nullptr : a.m + t.start;
            float v4[4], x4[4];
            if (full) {
                load4(vb, k0, v4);
                load4(xb, k0, x4);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4[q] = (k0 + q < (uint32_t)t.len) ? vb[k0 + q] : 1.0f;
                    x4[q] = (k0 + q < (uint32_t)t.len) ? xb[k0 + q] : 0.0f;
                }
            }
            float xn[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float upd = q4[q] / (sqrtf(v4[q]) + a.eps) + a.wd * x4[q];
                xn[q] = x4[q] - a.lr * upd;
            }
            if (full) {
                if (MODE != kUpdatePM) store4(mb, k0, q4);
                store4(eb, k0, e4);
                store4(xb, k0, xn);
                if (XB) {
                    uint2 pk;
                    pk.x = float_to_bf16_bits(xn[0]) | (float_to_bf16_bits(xn[1]) << 16);
                    pk.y = float_to_bf16_bits(xn[2]) | (float_to_bf16_bits(xn[3]) << 16);
                    st_stream(reinterpret_cast<uint2 *>(a.xb + t.start + k0), pk);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < (uint32_t)t.len) {
                        if (MODE != kUpdatePM) mb[k0 + q] = q4[q];
                        eb[k0 + q] = e4[q];
                        xb[k0 + q] = xn[q];
                        if (XB) a.xb[t.start + k0 + q] = (uint16_t)float_to_bf16_bits(xn[q]);
                    }
            }
        }
    }
}

// Pass-1 stores c where e was (e is fully rewritten by pass 2).
__device__ __forceinline__ void tile_store_c(const CompressArgs &a, const TileDesc &t, const float (&c)[kPerThread]) {
    const bool full = tile_full(a, t);
    float *eb = a.e + t.start;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        if (full) {
            *reinterpret_cast<float4 *>(eb + k0) = make_float4(c[4 * r], c[4 * r + 1], c[4 * r + 2], c[4 * r + 3]);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (k0 + q < (uint32_t)t.len) eb[k0 + q] = c[4 * r + q];
        }
    }
}

__device__ __forceinline__ void tile_load_c(const CompressArgs &a, const TileDesc &t, float (&c)[kPerThread]) {
    const bool full = tile_full(a, t);
    const float *eb = a.e + t.start;
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const uint32_t k0 = lane_k0(r);
        if (full) {
            const float4 cc = ld_stream(reinterpret_cast<const float4 *>(eb + k0));
            c[4 * r] = cc.x; c[4 * r + 1] = cc.y; c[4 * r + 2] = cc.z; c[4 * r + 3] = cc.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) c[4 * r + q] = (k0 + q < (uint32_t)t.len) ? eb[k0 + q] : 0.0f;
        }
    }
}

// Waves per SIMD the one-pass kernel is built for: six, five for the server tiles,
// whose staged worker words and fp64 sums need more registers than six waves leave.
constexpr int kOnepassWavesPerSimd = 6;
constexpr int kServerWavesPerSimd = 5;
constexpr int kMaxW = 1024;

// c of a posted tile waits in LDS (each thread reads back only what it wrote).
__device__ __forceinline__ void park_c(float4 *s, const float (&c)[kPerThread]) {
#pragma unroll
    for (int r = 0; r < kGroups; ++r)
        s[r * kBlock + threadIdx.x] = make_float4(c[4 * r], c[4 * r + 1], c[4 * r + 2], c[4 * r + 3]);
}
__device__ __forceinline__ void unpark_c(const float4 *s, float (&c)[kPerThread]) {
#pragma unroll
    for (int r = 0; r < kGroups; ++r) {
        const float4 v = s[r * kBlock + threadIdx.x];
        c[4 * r] = v.x;
        c[4 * r + 1] = v.y;
        c[4 * r + 2] = v.z;
        c[4 * r + 3] = v.w;
    }
}

// ------------------------------------------------------------- kernels
// One pass, persistent: the grid is at most the number of workgroups the device
// holds at once (its resident capacity for this kernel), so on an otherwise idle
// device every workgroup is resident from the start; a workgroup that has to wait
// for a slot (another stream's kernel holding CUs) becomes resident when that
// kernel's workgroups retire, since none of them waits on this kernel.
// Workgroup b takes list positions b, b+G, b+2G, ... and keeps kDepth tiles in
// flight: it computes and posts tile i+kDepth-1 (c parked in LDS) before it waits
// for tile i's chunk scale and finishes tile i, so the chunk-norm exchange
// overlaps streaming.  Termination: a workgroup posts tile i+kDepth-1 only after
// finishing tile i-1; if a chunk spans at most kDepth*G list positions, every
// workgroup has posted all its tiles of a chunk before it waits on that chunk,
// so the lowest unfinished chunk always completes.
constexpr int kDepth = 3;

// Tables the kernel only reads (tile list, tile and chunk descriptors) are read
// through the constant address space: their addresses are uniform, so the loads go
// through the scalar cache into scalar registers and no vector-memory wait (which
// would also wait for the previous tile's stores) stands before a tile's data loads.
__device__ __forceinline__ int32_t ld_table(const int32_t *p) {
    return *(const __attribute__((address_space(4))) int32_t *)p;
}
__device__ __forceinline__ TileDesc ld_table(const TileDesc *p) {
    typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
    static_assert(sizeof(TileDesc) == sizeof(i32x8_t), "tile descriptor is eight words");
    const i32x8_t v = *(const __attribute__((address_space(4))) i32x8_t *)p;
    TileDesc t;
    __builtin_memcpy(&t, &v, sizeof t);
    return t;
}
__device__ __forceinline__ ChunkDesc ld_table(const ChunkDesc *p) {
    typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
    static_assert(sizeof(ChunkDesc) == sizeof(i32x4_t), "chunk descriptor is four words");
    const i32x4_t v = *(const __attribute__((address_space(4))) i32x4_t *)p;
    ChunkDesc c;
    __builtin_memcpy(&c, &v, sizeof c);
    return c;
}

// The tiles a workgroup produces, in order.  With AHEAD the next one's descriptor
// is loaded a produce step before it is used and the list entry of the one after it
// two steps before, so a tile starts with its descriptor already in registers
// (compress-only worker on 64M 0.228 -> 0.220 ms, server 0.293 -> 0.290 ms).  The
// update modes load each descriptor with vector loads when its tile starts: they
// are bound by their bytes, and both the scalar registers held ahead and scalar
// loads alone made their step 0.5% slower.
struct TileQueue {
    int b, G, mine;
    int id0;      // next tile to produce
    TileDesc t0;  // its descriptor
    int id1;      // the tile after it
};

template <bool AHEAD>
__device__ __forceinline__ TileQueue tile_queue(const CompressArgs &a, int b, int G, int mine) {
    TileQueue q{b, G, mine, 0, TileDesc{}, 0};
    if (!AHEAD) return q;
    if (mine > 0) {
        q.id0 = ld_table(a.list + b);
        q.t0 = ld_table(a.tiles + q.id0);
    }
    if (mine > 1) q.id1 = ld_table(a.list + b + G);
    return q;
}

// Takes the tile at position p (the next one) and loads ahead for positions p+1, p+2.
template <bool AHEAD>
__device__ __forceinline__ void tile_queue_pop(const CompressArgs &a, TileQueue &q, int p, int &id, TileDesc &t) {
    if (!AHEAD) {
        id = a.list[q.b + p * q.G];
        t = a.tiles[id];
        return;
    }
    id = q.id0;
    t = q.t0;
    if (p + 1 < q.mine) {
        q.id0 = q.id1;
        q.t0 = ld_table(a.tiles + q.id1);
    }
    if (p + 2 < q.mine) q.id1 = ld_table(a.list + q.b + (p + 2) * q.G);
}

// Modes that load tile descriptors ahead (the light ones: compress-only and server).
constexpr bool loads_ahead(int mode) { return mode == kCompressOnly || is_server(mode) || mode == kCompressPM; }

template <int MODE, int GT>
__device__ __forceinline__ Posted produce(const CompressArgs &a, int tile_id, const TileDesc &t, float4 *slot_c,
                                          double *s_wscale_d, uint32_t *s_words, DD *s_red, uint32_t *s_u32,
                                          double *s_total) {
    ChunkDesc ch{};
    if (loads_ahead(MODE)) ch = ld_table(a.chunks + t.chunk);   // needed at the post, loaded now
    float c[kPerThread];
    tile_compute_c<MODE, GT>(a, t, c, s_wscale_d, s_words);
    tile_store_bits(a, t, c);
    park_c(slot_c, c);
    return post_tile<true>(a, tile_id, t.chunk, loads_ahead(MODE) ? &ch : nullptr, tile_sum_squares(c, s_red), s_red,
                           s_u32, s_total);
}

template <int MODE, int GT, bool XB>
__global__ __launch_bounds__(kBlock, is_server(MODE) ? kServerWavesPerSimd : kOnepassWavesPerSimd) void
k_compress_onepass(CompressArgs a) {
    __shared__ float4 s_c[kDepth][kGroups * kBlock];
    __shared__ TileDesc s_tile[kDepth];
    __shared__ Posted s_post[kDepth];
    __shared__ DD s_red[kWaves];
    __shared__ uint32_t s_u32[2];
    __shared__ double s_total;
    __shared__ double s_wscale_d[is_server(MODE) ? kServerLdsDoubles : 1];
    __shared__ __align__(16) uint32_t s_words[is_server(MODE) ? kWBatch * kTileWords : 1];
    const int G = (int)gridDim.x;
    // Workgroups are dispatched to the eight XCDs in turn; outside the server stage
    // the ones on one XCD take consecutive list positions (one-pass BERT-Large step
    // 1.80 -> 1.78 ms; the server tiles were 3% slower with it).  Any bijection of
    // the workgroup ids keeps the progress argument above.
    const bool xcd_runs = !is_server(MODE) && (G & 7) == 0;
    const int b = xcd_runs ? (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int mine = a.list_len > b ? (a.list_len - b + G - 1) / G : 0;  // tiles of this workgroup
    TileQueue q = tile_queue<loads_ahead(MODE)>(a, b, G, mine);
    // prologue: post the first kDepth-1 tiles
    for (int i = 0; i < kDepth - 1 && i < mine; ++i) {
        int id;
        TileDesc t;
        tile_queue_pop<loads_ahead(MODE)>(a, q, i, id, t);
        const Posted r = produce<MODE, GT>(a, id, t, s_c[i], s_wscale_d, s_words, s_red, s_u32, &s_total);
        if (threadIdx.x == 0) {
            s_tile[i] = t;
            s_post[i] = r;
        }
    }
    for (int i = 0; i < mine; ++i) {
        const int ahead = i + kDepth - 1;
        if (ahead < mine) {
            int id;
            TileDesc t;
            tile_queue_pop<loads_ahead(MODE)>(a, q, ahead, id, t);
            const int sl = ahead % kDepth;
            const Posted r = produce<MODE, GT>(a, id, t, s_c[sl], s_wscale_d, s_words, s_red, s_u32, &s_total);
            if (threadIdx.x == 0) {
                s_tile[sl] = t;
                s_post[sl] = r;
            }
        }
        __syncthreads();
        const int sl = i % kDepth;
        const TileDesc t = s_tile[sl];
        const Posted r = s_post[sl];
        const float scale = wait_scale(a, t.chunk, r, s_u32);
        float c[kPerThread];
        unpark_c(s_c[sl], c);
        tile_finish<MODE, XB>(a, t, c, scale);
    }
}

// Two passes for chunks too large for the one-pass kernel: pass 1 stores c in
// place of e, its sign words and its partial; a per-chunk kernel sums the
// partials; pass 2 finishes from c, v and x.
template <int MODE, int GT>
__global__ __launch_bounds__(kBlock) void k_compress_pass1(CompressArgs a) {
    __shared__ DD s_red[kWaves];
    __shared__ double s_wscale_d[is_server(MODE) ? kServerLdsDoubles : 1];
    __shared__ __align__(16) uint32_t s_words[is_server(MODE) ? kWBatch * kTileWords : 1];
    const int tile_id = a.list[blockIdx.x];
    const TileDesc t = a.tiles[tile_id];
    float c[kPerThread];
    tile_compute_c<MODE, GT>(a, t, c, s_wscale_d, s_words);
    tile_store_bits(a, t, c);
    tile_store_c(a, t, c);
    const double part = tile_sum_squares(c, s_red);
    if (threadIdx.x == 0) st_agent(a.slots + tile_id, tag_partial(part));
}

// One 1024-thread workgroup per two-pass chunk, 16 slot loads per thread in flight:
// a chunk of up to 16384 tiles is summed in one round of loads.
constexpr int kFinalizeThreads = 1024;

__global__ __launch_bounds__(kFinalizeThreads) void k_finalize_chunks(CompressArgs a, const int32_t *chunk_list) {
    __shared__ DD s_red[kFinalizeThreads / 64];
    __shared__ double s_total;
    const int chunk = chunk_list[blockIdx.x];
    const ChunkDesc ch = a.chunks[chunk];
    const double S = chunk_sum<kFinalizeThreads, 16>(a, ch, s_red, &s_total);
    if (threadIdx.x == 0) a.scales[chunk] = scale_of(S, ch.len);
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
template <int MODE, int GT, bool XB>
static onebit_status_t launch(const onebit_plan_s *p, CompressArgs a, hipStream_t stream) {
    const int base = is_server(MODE) ? kProfServerPass1 : kProfPass1;
    // Two-pass chunks first, pass 2 right after pass 1 so that the c it re-reads
    // is still in the memory-side cache; then the one-pass kernel for the rest.
    if (p->n_big > 0) {
        a.list = p->d_big_list;
        a.list_len = p->n_big;
        prof_before(base + 0, stream);
        hipLaunchKernelGGL((k_compress_pass1<MODE, GT>), dim3(p->n_big), dim3(kBlock), 0, stream, a);
        prof_after(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
        prof_before(kProfFinalize, stream);
        hipLaunchKernelGGL(k_finalize_chunks, dim3(p->n_big_chunks), dim3(kFinalizeThreads), 0, stream, a,
                           (const int32_t *)p->d_big_chunks);
        prof_after(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
        prof_before(base + 2, stream);
        hipLaunchKernelGGL((k_compress_pass2<MODE, XB>), dim3(p->n_big), dim3(kBlock), 0, stream, a);
        prof_after(stream);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    if (p->n_onepass > 0) {
        a.list = p->d_onepass_list;
        a.list_len = p->n_onepass;
        // Each variant runs with its own resident capacity; the plan's one-pass /
        // two-pass split was made for the smallest one, so kDepth * grid still
        // covers every one-pass chunk.  The caches are atomic: concurrent first
        // calls from several host threads compute and store the same value.
        static std::atomic<int32_t> cap_cache[64];
        const int dev = p->device;
        int32_t cap = (dev >= 0 && dev < 64) ? cap_cache[dev].load(std::memory_order_relaxed) : 0;
        if (cap <= 0) {
            int per_cu = 0, cus = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, reinterpret_cast<const void *>(&k_compress_onepass<MODE, GT, XB>), kBlock, 0) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                return ONEBIT_ERR_HIP;
            cap = per_cu * cus;
            if (dev >= 0 && dev < 64) cap_cache[dev].store(cap, std::memory_order_relaxed);
        }
        if (cap < p->resident_capacity) return ONEBIT_ERR_HIP;
        int grid = p->n_onepass < cap ? p->n_onepass : cap;
        const int32_t user_cap = g_grid_cap.load(std::memory_order_relaxed);
        if (user_cap > 0 && user_cap < grid) grid = user_cap;
        // the progress argument needs every one-pass chunk within kDepth * grid
        // consecutive list positions
        if ((int64_t)kDepth * grid < (int64_t)p->max_onepass_chunk_tiles) return ONEBIT_ERR_INVALID;
        prof_before(base + 1, stream);
        hipLaunchKernelGGL((k_compress_onepass<MODE, GT, XB>), dim3(grid), dim3(kBlock), 0, stream, a);
        prof_after(stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    return ONEBIT_OK;
}

static int occupancy_of(const void *fn) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kBlock, 0) != hipSuccess) return 0;
    return blocks;
}

int32_t onepass_depth() { return kDepth; }

int32_t resident_capacity(int device) {
    static std::atomic<int32_t> cached[64];
    if (device >= 0 && device < 64) {
        const int32_t c = cached[device].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
    const void *fns[] = {
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradF32, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradBF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradBF16, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdate, kGradF16, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressOnly, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressOnly, kGradBF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressOnly, kGradF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kServer, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kServerWide, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradF32, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradBF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradBF16, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kUpdatePM, kGradF16, true>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressPM, kGradF32, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressPM, kGradBF16, false>),
        reinterpret_cast<const void *>(&k_compress_onepass<kCompressPM, kGradF16, false>),
    };
    int per_cu = 1 << 30;
    for (const void *f : fns) {
        const int b = occupancy_of(f);
        per_cu = b < per_cu ? b : per_cu;
    }
    const int32_t cap = per_cu > 0 ? per_cu * cus : 0;
    if (device >= 0 && device < 64) cached[device].store(cap, std::memory_order_relaxed);
    return cap;
}

// ------------------------------------------- scratch of the allocation-free call
// The workspace of onebit_compress_update_static lives in the library's own device
// memory: an error word, one publish word per chunk and one partial slot per tile
// for plans with chunks + tiles < kScratchWords (8 MiB; each device the library
// runs on holds its own copy until the process ends).  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr int64_t kScratchWords = int64_t(1) << 20;
static __device__ __align__(256) uint64_t scratch[kScratchWords];

static std::mutex g_scratch_mu;
static uint64_t *g_scratch_ptr[64];

static onebit_status_t scratch_address(int dev, uint64_t **out) {
    if (dev < 0 || dev >= 64) return ONEBIT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return ONEBIT_ERR_HIP;
        }
        g_scratch_ptr[dev] = static_cast<uint64_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return ONEBIT_OK;
}

__global__ __launch_bounds__(256) void k_clear_words(uint64_t *p, int64_t words) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void k_copy_word(uint64_t *dst, const uint64_t *src) {
    if (threadIdx.x == 0) *dst = src ? ld_agent(src) : 0;
}

// What the allocation-free call adds around the shared dispatch: the scratch words
// it clears before the kernels run, and the device word that receives the error
// word after them (nullable).
struct ScratchUse {
    int64_t clear_words;
    uint64_t *status_out;
};

}  // namespace onebit

using namespace onebit;

// Validation and dispatch shared by the fp32-momentum and the packed-momentum
// entry points (exactly one of m and m_bits is given), and by the allocation-free
// call (sc non-null: workspace is the scratch).
static onebit_status_t compress_entry(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype, float *m,
                                      const uint32_t *m_bits, const float *m_scales, const uint8_t *m_mask,
                                      float *e, const float *v,
                                      float *x, uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                      double beta1, double eps, double weight_decay, void *workspace,
                                      void *stream, const ScratchUse *sc = nullptr);

static onebit_status_t dispatch_compress(const onebit_plan_s *plan, const CompressArgs &a, onebit_dtype_t g_dtype,
                                         bool packed, bool update, bool xb, hipStream_t s);

static onebit_status_t compress_entry(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype, float *m,
                                      const uint32_t *m_bits, const float *m_scales, const uint8_t *m_mask,
                                      float *e, const float *v,
                                      float *x, uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                      double beta1, double eps, double weight_decay, void *workspace,
                                      void *stream, const ScratchUse *sc) {
    if (!plan) return ONEBIT_ERR_INVALID;
    if (g_dtype != ONEBIT_F32 && g_dtype != ONEBIT_BF16 && g_dtype != ONEBIT_F16) return ONEBIT_ERR_INVALID;
    const bool packed = m_bits != nullptr || m_scales != nullptr;
    const bool update = (v != nullptr) || (x != nullptr);
    if (update && (!v || !x)) return ONEBIT_ERR_INVALID;
    if (!update && x_bf16) return ONEBIT_ERR_INVALID;
    if (m_mask && !packed) return ONEBIT_ERR_INVALID;
    if (sc && sc->status_out && !aligned_to(sc->status_out, 8)) return ONEBIT_ERR_ALIGN;
    if (plan->n_chunks == 0) {
        if (!sc || !sc->status_out) return ONEBIT_OK;
        hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), sc->status_out,
                           nullptr);
        return hip_status(hipGetLastError());
    }
    if (!scales || !workspace) return ONEBIT_ERR_INVALID;
    if (packed && (!m_scales || (plan->n > 0 && !m_bits) || m_scales == scales || (m_bits && m_bits == bits)))
        return ONEBIT_ERR_INVALID;
    if (plan->n > 0 && (!g || (!packed && !m) || !e || !bits)) return ONEBIT_ERR_INVALID;
    const void *vec[] = {g, m, e, v, x, x_bf16};
    for (const void *q : vec)
        if (q && !aligned16(q)) return ONEBIT_ERR_ALIGN;
    if (!aligned_to(bits, 4) || !aligned_to(scales, 4) || !aligned_to(workspace, 8)) return ONEBIT_ERR_ALIGN;
    if (!aligned_to(m_bits, 4) || !aligned_to(m_scales, 4) || !aligned_to(m_mask, 4)) return ONEBIT_ERR_ALIGN;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;

    CompressArgs a{};
    a.tiles = plan->d_tiles;
    a.chunks = plan->d_chunks;
    a.mask_iv = plan->d_mask_iv;
    a.aligned = plan->aligned ? 1 : 0;
    a.g = g;
    a.m = m;
    a.m_bits = m_bits;
    a.m_scales = m_scales;
    a.m_mask = m_mask;
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
    a.publish = ws.publish;
    a.slots = ws.slots;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (sc) {
        const int64_t blocks = std::min<int64_t>((sc->clear_words + 255) / 256, 1024);
        hipLaunchKernelGGL(k_clear_words, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s,
                           static_cast<uint64_t *>(workspace), sc->clear_words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_status(e);
    }
    onebit_status_t st = dispatch_compress(plan, a, g_dtype, packed, update, x_bf16 != nullptr, s);
    if (sc && sc->status_out) {
        hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(64), 0, s, sc->status_out,
                           static_cast<const uint64_t *>(workspace));
        const hipError_t e = hipGetLastError();
        if (st == ONEBIT_OK && e != hipSuccess) st = hip_status(e);
    }
    return st;
}

static onebit_status_t dispatch_compress(const onebit_plan_s *plan, const CompressArgs &a, onebit_dtype_t g_dtype,
                                         bool packed, bool update, bool xb, hipStream_t s) {
    if (packed && !update) {
        switch (g_dtype) {
            case ONEBIT_BF16: return launch<kCompressPM, kGradBF16, false>(plan, a, s);
            case ONEBIT_F16: return launch<kCompressPM, kGradF16, false>(plan, a, s);
            default: return launch<kCompressPM, kGradF32, false>(plan, a, s);
        }
    }
    if (packed) {
        switch (g_dtype) {
            case ONEBIT_BF16:
                return xb ? launch<kUpdatePM, kGradBF16, true>(plan, a, s)
                          : launch<kUpdatePM, kGradBF16, false>(plan, a, s);
            case ONEBIT_F16:
                return xb ? launch<kUpdatePM, kGradF16, true>(plan, a, s)
                          : launch<kUpdatePM, kGradF16, false>(plan, a, s);
            default:
                return xb ? launch<kUpdatePM, kGradF32, true>(plan, a, s)
                          : launch<kUpdatePM, kGradF32, false>(plan, a, s);
        }
    }
    switch (g_dtype) {
        case ONEBIT_BF16:
            if (!update) return launch<kCompressOnly, kGradBF16, false>(plan, a, s);
            return xb ? launch<kUpdate, kGradBF16, true>(plan, a, s) : launch<kUpdate, kGradBF16, false>(plan, a, s);
        case ONEBIT_F16:
            if (!update) return launch<kCompressOnly, kGradF16, false>(plan, a, s);
            return xb ? launch<kUpdate, kGradF16, true>(plan, a, s) : launch<kUpdate, kGradF16, false>(plan, a, s);
        default:
            if (!update) return launch<kCompressOnly, kGradF32, false>(plan, a, s);
            return xb ? launch<kUpdate, kGradF32, true>(plan, a, s) : launch<kUpdate, kGradF32, false>(plan, a, s);
    }
}

extern "C" onebit_status_t onebit_compress_update(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                                  float *m, float *e, const float *v, float *x,
                                                  uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                                  double beta1, double eps, double weight_decay,
                                                  void *workspace, void *stream) {
    return compress_entry(plan, g, g_dtype, m, nullptr, nullptr, nullptr, e, v, x, x_bf16, bits, scales, lr, beta1,
                          eps, weight_decay, workspace, stream);
}

extern "C" onebit_status_t onebit_compress_update_packed(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                                         const uint32_t *m_bits, const float *m_scales,
                                                         const uint8_t *m_mask, float *e, const float *v, float *x,
                                                         uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                                         double beta1, double eps, double weight_decay,
                                                         void *workspace, void *stream) {
    if (!m_scales) return ONEBIT_ERR_INVALID;
    return compress_entry(plan, g, g_dtype, nullptr, m_bits, m_scales, m_mask, e, v, x, x_bf16, bits, scales, lr,
                          beta1, eps, weight_decay, workspace, stream);
}

extern "C" onebit_status_t onebit_compress_update_static(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                                         float *m, float *e, const float *v, float *x,
                                                         uint16_t *x_bf16, uint32_t *bits, float *scales,
                                                         double lr, double beta1, double eps, double weight_decay,
                                                         uint64_t *wait_status, void *stream) {
    if (!plan) return ONEBIT_ERR_INVALID;
    const int64_t words = 1 + plan->n_chunks + plan->n_tiles;
    if (words > kScratchWords) return ONEBIT_ERR_NOMEM;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return ONEBIT_ERR_INVALID;
    uint64_t *ws = nullptr;
    const onebit_status_t st = scratch_address(dev, &ws);
    if (st != ONEBIT_OK) return st;
    const ScratchUse sc{words, wait_status};
    return compress_entry(plan, g, g_dtype, m, nullptr, nullptr, nullptr, e, v, x, x_bf16, bits, scales, lr, beta1,
                          eps, weight_decay, ws, stream, &sc);
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
    a.w_pow2_scale = (W & (W - 1)) == 0 ? 1.0 / (double)W : 0.0;
    a.plan_words = plan->words;
    a.n_chunks = plan->n_chunks;
    a.m_out = m_out;
    a.bits = server_bits;
    a.scales = server_scales;
    const WorkspaceView ws = workspace_view(workspace, plan->n_chunks);
    a.err = ws.err;
    a.publish = ws.publish;
    a.slots = ws.slots;
    a.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
    if (W > kWBatch) return launch<kServerWide, kGradF32, false>(plan, a, static_cast<hipStream_t>(stream));
    return launch<kServer, kGradF32, false>(plan, a, static_cast<hipStream_t>(stream));
}

extern "C" void onebit_set_spin_limit(uint32_t limit) {
    g_spin_limit.store(limit ? limit : kSpinLimit, std::memory_order_relaxed);
}

extern "C" void onebit_set_grid_cap(int32_t cap) { g_grid_cap.store(cap > 0 ? cap : 0, std::memory_order_relaxed); }

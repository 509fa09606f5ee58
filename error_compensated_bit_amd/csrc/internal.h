// internal.h -- host-side structures shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "onebit.h"

namespace onebit {

// One tile = up to kTile consecutive elements of one chunk, starting at a
// chunk-relative offset that is a multiple of kTile (so of 32: its first packed
// word is whole).
struct TileDesc {
    int64_t start;    // first element (absolute)
    int64_t word;     // first packed word (absolute)
    int32_t len;      // elements, 0..kTile (0 only for an empty chunk)
    int32_t chunk;    // owning chunk
    int32_t mask_lo;  // masked intervals [mask_lo, mask_hi) touching the tile;
    int32_t mask_hi;  // mask_lo == -1: the whole tile is masked
};

struct ChunkDesc {
    int64_t len;
    int32_t first_tile;
    int32_t ntiles;
};

// Workspace layout (all 8-byte words, zero = ready):
//   [0]                      error word (non-zero after a spin timeout)
//   [1 .. 1+n_chunks)        per chunk: published {epoch:32 | scale bits:32}
//   [.. + n_tiles)           per tile: tagged fp64 partial sum of squares (0 = empty)
struct WorkspaceView {
    uint64_t *err;
    uint64_t *publish;
    uint64_t *slots;
};

}  // namespace onebit

struct onebit_plan_s {
    int device = 0;
    int64_t n = 0;
    int64_t n_chunks = 0;
    int64_t n_tiles = 0;
    int64_t words = 0;
    int64_t n_mask_iv = 0;
    int32_t max_chunk_tiles = 0;
    bool aligned = true;         // every chunk starts on a multiple of 4 elements
    onebit::TileDesc *d_tiles = nullptr;
    onebit::ChunkDesc *d_chunks = nullptr;
    int64_t *d_mask_iv = nullptr;     // 2*n_mask_iv: [a, b) pairs, sorted, disjoint
    int32_t *d_onepass_list = nullptr;  // tiles of chunks the one-pass kernel takes
    int32_t *d_big_list = nullptr;    // tiles of the other chunks (two-pass)
    int32_t *d_big_chunks = nullptr;  // the two-pass chunks
    int32_t n_onepass = 0;
    int32_t n_big = 0;
    int32_t n_big_chunks = 0;
    int32_t resident_capacity = 0;    // resident workgroups the split was made for
    int32_t max_onepass_chunk_tiles = 0;  // tiles of the largest one-pass chunk
};

namespace onebit {

size_t workspace_bytes_for(int64_t n_chunks, int64_t n_tiles);
WorkspaceView workspace_view(void *ws, int64_t n_chunks);
bool aligned16(const void *p);
bool aligned_to(const void *p, uintptr_t bytes);
onebit_status_t hip_status(hipError_t e);

// Largest number of co-resident workgroups of the one-pass compress kernels on this
// device (the smallest over their variants), and the number of tiles each
// workgroup keeps in flight.
int32_t resident_capacity(int device);
int32_t onepass_depth();

// Launch timing (diagnostics): while a profiling session is open every kernel
// launch of the library is bracketed by two events on its stream.
enum ProfClass {
    kProfWarmup = 0,
    kProfPass1 = 1,
    kProfOnepass = 2,
    kProfPass2 = 3,
    kProfQuantize = 4,
    kProfDequantize = 5,
    kProfServerPass1 = 6,
    kProfServerOnepass = 7,
    kProfServerPass2 = 8,
    kProfFinalize = 9,
    kProfMomentumUpdate = 10,
    kProfQsgdQuantize = 11,
    kProfQsgdReduce = 12,
    kProfLocoQuantize = 13,
    kProfClasses = 14
};
void prof_before(int cls, hipStream_t s);
void prof_after(hipStream_t s);

}  // namespace onebit

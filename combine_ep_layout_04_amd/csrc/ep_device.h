// ep_device.h -- device-side helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of a gfx950 vector memory instruction: bit 0 sc0,
// bit 1 nt, bit 4 sc1.  Rows written once and not read again by the kernel
// go out with sc1 | nt (device scope, non-temporal): they stream past the
// caches.  On the dispatch pattern this measured about 2% faster than nt
// alone with cold caches and 3% back to back.
constexpr int kCpolNT = 2;
constexpr int kCpolStream = 16 | 2;

// Raw buffer resource over `bytes` bytes at p (stride 0; the 32-bit data
// format word of the gfx9 resource descriptor).  Accesses past `bytes`
// read 0 and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of a write-once row.
__device__ __forceinline__ void store_row16(__amdgpu_buffer_rsrc_t rs, int off, const uint4& v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCpolStream);
}

// 16 bytes at byte offset `off` (0 past the resource's end), cache policy
// `cpol`.
template <int cpol>
__device__ __forceinline__ uint4 load_row16(__amdgpu_buffer_rsrc_t rs, int off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, cpol));
}

// Row tiles.  The row-copying kernels split every row into tiles of
// kTileLanes 16-byte vectors (2 KiB) and give each workgroup of kTileLanes
// lanes one tile, one vector per lane, so a workgroup issues one store per
// destination row and exits.  On MI355X, streams written by workgroups that
// store one or two 2 KiB pieces each ran at 6.3-6.5 TB/s, against
// 5.2-5.3 TB/s when each workgroup wrote 7 to 56 of them in turn.
constexpr int kTileLanes = 128;

__host__ __device__ inline int tiles_per_row(int nvec) { return (nvec + kTileLanes - 1) / kTileLanes; }

// Rows whose last 128-lane tile would be at most half full (units mod 128 in
// 1..64, for rows of more than 128 units) take 64-lane tiles: 64 fewer
// lanes per row launched.  Measured on MI355X (T=8192, caches emptied
// before each launch, interleaved A/B rounds on one machine), 64-lane tiles
// were faster on every such row tried: the combine (k=8) by 7-12% at hidden
// 1152-1536 and 3.5% at 3584, the combine over 8 ranks by 3-12% at
// 1152-1536 and 3.4% at 3584, the 8-bit cast by 11% at 3072 and 1-2% at
// 7168; within 1% at hidden 2560, 5120 and 5632.  On rows of whole 128-lane
// tiles 64-lane ones were up to 2% slower.
__host__ __device__ inline bool narrow_tiles(int units)
{
    const int tail = units % kTileLanes;
    return units > kTileLanes && tail != 0 && tail <= kTileLanes / 2;
}

// When a dispatch (one row to several destinations) is tiled.  Measured
// against one workgroup per token on MI355X (T 2048-8192, k 4 and 8,
// hidden 1536-4096, caches emptied before each launch):
//   - rows of 512 vectors and more: tiles as fast or faster everywhere;
//   - rows of 256 or 384 vectors (whole tiles): tiles 3-7% faster once the
//     dispatch writes at least 2^23 vectors (134 MB), up to 19% slower below;
//   - rows that end in a partial tile (192 vectors): tiles 7-11% slower.
constexpr int kMinTiledDispatchVectors = 512;
constexpr int64_t kMinTiledDispatchWork = int64_t(1) << 23;   // vectors written

__host__ __device__ inline bool tile_dispatch(int nvec, int64_t rows_written)
{
    return nvec >= kMinTiledDispatchVectors ||
           (nvec >= 2 * kTileLanes && nvec % kTileLanes == 0 &&
            rows_written * nvec >= kMinTiledDispatchWork);
}

// Workgroups are dispatched to the 8 XCDs round robin (workgroup b runs on
// XCD b % 8), and each XCD has its own L2.  When `per_tile` workgroups
// read the same tile, this maps workgroup b to (tile, member) so that a
// tile's workgroups run back to back on one XCD and all but the first find
// it in that L2: XCD x takes tiles x, x + 8, x + 16, ...  Returns false for
// the workgroups of the padding past num_tiles (the grid is a multiple of
// 8 * per_tile).
__device__ __forceinline__ bool xcd_tile(int64_t b, int per_tile, int64_t num_tiles,
                                         int64_t& tile, int& member)
{
    const int64_t s = b >> 3;
    tile = (s / per_tile) * 8 + (b & 7);
    member = (int)(s % per_tile);
    return tile < num_tiles;
}

}  // namespace ep

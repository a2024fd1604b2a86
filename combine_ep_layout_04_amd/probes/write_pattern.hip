// write_pattern.hip -- measurement kernels for the bf16 dispatch's access
// pattern (built as libep_probe.so; not part of the C ABI).  They separate
// what the dispatch's scattered row writes cost from what reading the
// tokens costs, at the dispatch's own shape:
//
//   stores_only_tile_kernel  the tiled dispatch's grid, XCD order and slot
//                            map, storing a constant instead of x (no loads
//                            besides the slots);
//   write_stream_kernel      the same bytes written in destination order,
//                            one-shot workgroups of 2 KiB or 4 KiB, or
//                            14 KiB per workgroup in turn;
//   read_x_kernel            x read once, 2 KiB per workgroup;
//   gather_kernel            the dispatch in destination order: each
//                            workgroup writes one 2 KiB tile of a receive row
//                            and loads it from x[src[row]] (x read k times);
//   order_row_kernel         whole receive rows, one workgroup each, visited
//                            in a given order (token order, destination
//                            order, or windows of tokens expert by expert),
//                            each loaded from x[src[row]]; or, XCD-aware,
//                            one list of rows per XCD (workgroup b runs on
//                            XCD b mod 8), so that a window's rows, and its
//                            tokens' re-reads, stay in one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"

using namespace ep;

namespace {

__global__ __launch_bounds__(kTileLanes)
void stores_only_tile_kernel(int nvec, int k, int tpr, int64_t num_tiles, int groups,
                             const int32_t* __restrict__ slot, uint4* __restrict__ recv)
{
    int64_t tile;
    int g;
    if (!xcd_tile(blockIdx.x, groups, num_tiles, tile, g)) return;
    const int64_t t = tile / tpr;
    const int p = (int)(tile - t * tpr);
    const int tid = threadIdx.x, lane = tid & 63;
    const int j0 = g * 4;
    const int32_t sl = lane < 4 && j0 + lane < k ? slot[t * k + j0 + lane] : -1;
    int32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_readlane(sl, q);
    const int v = p * kTileLanes + tid;
    const uint4 d = make_uint4((uint32_t)tile, (uint32_t)tid, 0x5A5A5A5Au, (uint32_t)g);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (r[q] >= 0 && v < nvec) store_row16(buffer_rsrc(recv + (int64_t)r[q] * nvec, nvec * 16), v * 16, d);
}

// workgroup b writes vectors [b*NL*VPL, (b+1)*NL*VPL) of dst, VPL stores per lane in turn
template <int NL, int VPL>
__global__ __launch_bounds__(NL)
void write_stream_kernel(uint4* __restrict__ dst, int64_t nvec_total)
{
    const int64_t base = (int64_t)blockIdx.x * NL * VPL;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(dst + base, NL * VPL * 16);
    const uint4 d = make_uint4(blockIdx.x, threadIdx.x, 1u, 2u);
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
        const int64_t v = base + u * NL + threadIdx.x;
        if (v < nvec_total) store_row16(rs, (int)(v - base) * 16, d);
    }
}

__global__ __launch_bounds__(kTileLanes)
void read_x_kernel(const uint4* __restrict__ x, int64_t nvec_total, uint32_t* sink)
{
    const int64_t v = (int64_t)blockIdx.x * kTileLanes + threadIdx.x;
    const uint4 d = v < nvec_total ? x[v] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t h = d.x ^ d.y ^ d.z ^ d.w;
    if (h == 0x12345678u) sink[0] = h;   // keeps the loads; the sink is a 4-byte buffer
}

__global__ __launch_bounds__(kTileLanes)
void gather_kernel(const uint4* __restrict__ x, int nvec, int tpr, int n_rows,
                   const int32_t* __restrict__ src, uint4* __restrict__ recv)
{
    const int b = blockIdx.x;
    const int r = b / tpr, p = b - r * tpr;
    if (r >= n_rows) return;
    const int t = src[r];
    const int v = p * kTileLanes + threadIdx.x;
    const uint4 d = load_row16<0>(buffer_rsrc(x + (int64_t)t * nvec, nvec * 16), v * 16);
    if (v < nvec) store_row16(buffer_rsrc(recv + (int64_t)r * nvec, nvec * 16), v * 16, d);
}

// workgroup b copies receive row order[b] from x[src[order[b]]], the whole
// row (up to 8 vectors per lane) loaded before it is stored.  With per_xcd
// > 0, order is [8, per_xcd] and workgroup b takes entry b / 8 of list b % 8
// (entries of -1 pad the shorter lists).
__global__ __launch_bounds__(kTileLanes)
void order_row_kernel(const uint4* __restrict__ x, int64_t T, int nvec, int n_rows,
                      const int32_t* __restrict__ order, int per_xcd, const int32_t* __restrict__ src,
                      uint4* __restrict__ recv)
{
    const int at = per_xcd > 0 ? (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    const int r = __builtin_amdgcn_readfirstlane(order[at]);
    if (r < 0 || r >= n_rows) return;
    const int t = __builtin_amdgcn_readfirstlane(src[r]);
    if (t < 0 || t >= T) return;
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + (int64_t)t * nvec, nvec * 16);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(recv + (int64_t)r * nvec, nvec * 16);
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load_row16<0>(xs, (u * kTileLanes + (int)threadIdx.x) * 16);
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (u * kTileLanes + (int)threadIdx.x < nvec)
            store_row16(rs, (u * kTileLanes + (int)threadIdx.x) * 16, v[u]);
}
}  // namespace

// recv: [T*k, hidden/8] 16-byte vectors; slot: [T, k] rows of recv (or -1)
extern "C" int probe_stores_only(int64_t T, int hidden, int k, const int32_t* slot, void* recv,
                                 hipStream_t s)
{
    const int nvec = hidden / 8, tpr = (nvec + kTileLanes - 1) / kTileLanes, groups = (k + 3) / 4;
    const int64_t num_tiles = T * tpr, blocks = (num_tiles + 7) / 8 * 8 * groups;
    if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stores_only_tile_kernel, dim3((unsigned)blocks), dim3(kTileLanes), 0, s, nvec, k,
                       tpr, num_tiles, groups, slot, (uint4*)recv);
    return (int)hipGetLastError();
}

// dst: `bytes` bytes (a multiple of 16); piece_kib: 2, 4 or 14
extern "C" int probe_write_stream(void* dst, int64_t bytes, int piece_kib, hipStream_t s)
{
    const int64_t nv = bytes / 16;
    if (piece_kib == 2)
        hipLaunchKernelGGL((write_stream_kernel<128, 1>), dim3((unsigned)((nv + 127) / 128)), dim3(128), 0, s,
                           (uint4*)dst, nv);
    else if (piece_kib == 4)
        hipLaunchKernelGGL((write_stream_kernel<256, 1>), dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s,
                           (uint4*)dst, nv);
    else
        hipLaunchKernelGGL((write_stream_kernel<128, 7>), dim3((unsigned)((nv + 895) / 896)), dim3(128), 0, s,
                           (uint4*)dst, nv);
    return (int)hipGetLastError();
}

// x: `bytes` bytes (a multiple of 16); sink: 4 bytes
extern "C" int probe_read_x(const void* x, int64_t bytes, uint32_t* sink, hipStream_t s)
{
    const int64_t nv = bytes / 16;
    hipLaunchKernelGGL(read_x_kernel, dim3((unsigned)((nv + kTileLanes - 1) / kTileLanes)), dim3(kTileLanes),
                       0, s, (const uint4*)x, nv, sink);
    return (int)hipGetLastError();
}

// src: [n_rows] source token of each receive row; recv: [n_rows, hidden]
extern "C" int probe_gather(const void* x, int hidden, int n_rows, const int32_t* src, void* recv,
                            hipStream_t s)
{
    const int nvec = hidden / 8, tpr = (nvec + kTileLanes - 1) / kTileLanes;
    if ((int64_t)n_rows * tpr > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(n_rows * tpr)), dim3(kTileLanes), 0, s,
                       (const uint4*)x, nvec, tpr, n_rows, src, (uint4*)recv);
    return (int)hipGetLastError();
}

// order: a permutation of [0, n_rows) (per_xcd == 0), or 8 lists of
// per_xcd entries, each a row or -1, together holding every row once;
// src: [n_rows] tokens in [0, T); rows of at most 8 * 128 vectors
// (hidden <= 8192)
extern "C" int probe_order_rows(const void* x, int64_t T, int hidden, int n_rows, const int32_t* order,
                                int per_xcd, const int32_t* src, void* recv, hipStream_t s)
{
    const int nvec = hidden / 8;
    if (nvec > 8 * kTileLanes || n_rows <= 0 || per_xcd < 0) return (int)hipErrorInvalidValue;
    const unsigned grid = per_xcd > 0 ? 8u * (unsigned)per_xcd : (unsigned)n_rows;
    hipLaunchKernelGGL(order_row_kernel, dim3(grid), dim3(kTileLanes), 0, s,
                       (const uint4*)x, T, nvec, n_rows, order, per_xcd, src, (uint4*)recv);
    return (int)hipGetLastError();
}

// ep_dispatch.hip -- permute token rows into the expert-grouped receive
// buffer (bf16 copy or OCP E4M3 cast with per-128-channel fp32 scales).
//
// Passages: NCCL EP page, nccl_ep.cc, ncclEpDispatch (bf16 tokens [T,
// hidden] with 16-byte rows; fp8 output with a scales tensor of hidden/128
// fp32 per token, scale block 128; dense-to-sparse step that hands each
// received row its top-k weight); DeepEP page, dispatch() returning recv_x
// and recv_topk_weights.
//
// Design (HBM-bound; no arithmetic worth a matrix core):
//   - bf16: one workgroup per (2 KiB row tile, group of up to 4 of the
//     token's slots), one 16-byte vector per lane: it loads its tile of x[t]
//     and stores it to the group's destination rows, at most 4 stores per
//     lane.  The ceil(k/4) workgroups of a tile run back to back on one XCD,
//     so x[t] comes from HBM once and the other loads hit that XCD's L2.
//     Against one workgroup per token (the row held in registers and
//     written to all k rows) this measured 200 us instead of 218 us at
//     T=8192, hidden 7168, k=8 with cold caches: workgroups that each write
//     a few 2 KiB pieces stream faster than ones that write 56 in turn.
//     Short rows (under 512 vectors, unless they are whole tiles and the
//     dispatch writes at least 2^23 vectors, or rows of 257-511 vectors
//     whose last tile would be at most half full, which take 64-lane
//     tiles), and grids past 2^31 workgroups, keep one workgroup per token;
//   - the slots a workgroup serves are wavefront-uniform (read into lanes,
//     then readlane), so the loop over destinations has no divergence;
//   - fp8: each lane owns 16 channels (a "unit": two 16-byte loads in, one
//     16-byte store out), so 8 aligned lanes hold one 128-channel block and
//     amax is an 8-lane reduction by DPP lane moves (no LDS traffic).  With row-major scales and rows
//     of more than 64 units, one 128-lane workgroup per (token, tile of 128
//     units, group of up to 4 slots; 8 on rows of at most 256 units), or
//     64-lane tiles where the last 128-lane tile would be at most half
//     full, with all of a token's workgroups back to back on one XCD
//     (its scale rows are written in pieces by several tiles, and those
//     pieces then meet in one L2); otherwise one 64-lane wavefront per
//     token.  The scale is a correctly rounded fp32 division.  Each quotient x / scale
//     must be the correctly rounded fp32 quotient too; instead of a full
//     division per element it uses Markstein's correction (P. Markstein,
//     "Computation of elementary functions on the IBM RISC System/6000
//     processor", IBM J. Res. Dev. 34(1), 1990): with y = RN(1/scale)
//     computed once, q0 = |x| * y, r = fma(-q0, scale, |x|) (exact),
//     q = fma(r, y, q0).  That q was checked to give the same code as the
//     correctly rounded quotient, in E4M3 (scale amax / 448) and in E5M2
//     (scale amax / 57344), for every bf16 amax >= 2^-80 and every bf16
//     |x| <= amax; blocks with a smaller, infinite or NaN amax take the
//     plain division.  The sign is applied after encoding |q|, so -0 stays
//     -0.  The E4M3 code comes from an integer round-to-nearest-even on the
//     fp32 bit pattern (written from the OCP E4M3 definition: bias 7,
//     largest finite 448, codes below 2^-6 are multiples of 2^-9).
//     In the per-token kernel the block scales of a pass are staged in LDS
//     and written with one coalesced store per destination row: scattered
//     4-byte scale stores interleaved with the code stores measured ~30%
//     slower.

#include <algorithm>

#include "ep_cast.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

// Lane j of every wavefront holds slot[t, j] (k <= 64); the destination
// loop reads it back with readlane, so each destination costs one scalar
// register read and no memory round trip.
__device__ __forceinline__ int32_t token_slots(const int32_t* s, int k)
{
    const int lane = threadIdx.x & 63;
    return lane < k ? s[lane] : -1;
}

__device__ __forceinline__ int32_t lane_value(int32_t v, int j)
{
    return __builtin_amdgcn_readlane(v, j);
}

// Destination rows are written once and not read again by this kernel:
// they go out as streaming buffer stores (store_row16: sc1 | nt), which
// measured ~12% faster than cached stores on MI355X back to back.

// Keeps a loaded vector in registers: without it the compiler may sink the
// load into the destination loop and read the source row k times.
__device__ __forceinline__ void keep(uint4& v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

template <int NT, int VPT>
__global__ __launch_bounds__(NT)
void dispatch_bf16_kernel(const uint4* __restrict__ x, int nvec, int k,
                          const int32_t* __restrict__ slot, const float* __restrict__ w,
                          uint4* __restrict__ recv, float* __restrict__ recv_w)
{
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* s = slot + t * k;
    const int32_t sl = token_slots(s, k);

    if (recv_w != nullptr && tid < k && sl >= 0) recv_w[sl] = w[t * k + tid];

    const uint4* xr = x + t * nvec;
    constexpr int kPass = NT * VPT;
    const int full = nvec / kPass;

    // whole passes: VPT 16-byte vectors per lane, no bounds checks
    for (int p = 0; p < full; ++p) {
        const int vb = p * kPass + tid;
        uint4 buf[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) buf[u] = xr[vb + u * NT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) keep(buf[u]);
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r < 0) continue;
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(recv + (int64_t)r * nvec, nvec * 16);
#pragma unroll
            for (int u = 0; u < VPT; ++u) store_row16(rs, (vb + u * NT) * 16, buf[u]);
        }
    }
    // ragged tail: one vector per lane.  The trip count is the same for
    // every lane, so lane_value always runs with the whole wavefront active
    // (it reads another lane's register, whose value is only kept for lanes
    // that are active); past the row end the load reads 0 and nothing is
    // stored.
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(xr, nvec * 16);
    for (int v0 = full * kPass; v0 < nvec; v0 += NT) {
        const int v = v0 + tid;
        uint4 d = load_row16<0>(xs, v * 16);
        keep(d);
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r >= 0 && v < nvec) store_row16(buffer_rsrc(recv + (int64_t)r * nvec, nvec * 16), v * 16, d);
        }
    }
}

// Tiled form: workgroup b maps (XCD-aware) to tile `tile` = (token t, tile
// p of its row) and slot group g (slots 4g .. 4g+3).
constexpr int kSlotsPerGroup = 4;

template <int NL>
__global__ __launch_bounds__(NL)
void dispatch_bf16_tile_kernel(const uint4* __restrict__ x, int nvec, int k, int tpr,
                               int64_t num_tiles, int groups, const int32_t* __restrict__ slot,
                               const float* __restrict__ w, uint4* __restrict__ recv,
                               float* __restrict__ recv_w)
{
    int64_t tile;
    int g;
    if (!xcd_tile(blockIdx.x, groups, num_tiles, tile, g)) return;
    const int64_t t = tile / tpr;
    const int p = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j0 = g * kSlotsPerGroup;
    // lanes 0..3 of each wavefront hold the group's slots
    const int32_t sl = lane < kSlotsPerGroup && j0 + lane < k ? slot[t * k + j0 + lane] : -1;
    if (recv_w != nullptr && p == 0 && tid < kSlotsPerGroup && sl >= 0)
        recv_w[sl] = w[t * k + j0 + tid];

    int32_t r[kSlotsPerGroup];
#pragma unroll
    for (int q = 0; q < kSlotsPerGroup; ++q) r[q] = lane_value(sl, q);
    const int v = p * NL + tid;             // past the row end (last tile) stores nothing
    uint4 d = load_row16<0>(buffer_rsrc(x + t * nvec, nvec * 16), v * 16);
    keep(d);
#pragma unroll
    for (int q = 0; q < kSlotsPerGroup; ++q)
        if (r[q] >= 0 && v < nvec) store_row16(buffer_rsrc(recv + (int64_t)r[q] * nvec, nvec * 16), v * 16, d);
}

// ---------------------------------------------------------------- fp8 ---

// One 64-lane wavefront per token.  A "unit" is 16 channels (two input
// vectors, one 16-byte output vector); a pass covers up to 64*VPT units and
// 8*VPT <= 64 blocks.  Units past the row end read zeros and store nothing
// (hidden is a multiple of 128, so an 8-lane block group is all in or all
// out).  Scales go out as fp32 (modes 0, 1) or bytes (mode 2), row-major
// [rows, nb] (sld == 0) or column-major [nb, sld] (block b of row r at
// b * sld + r).
template <int VPT, int FMT, int SM>
__global__ __launch_bounds__(64)
void dispatch_fp8_kernel(const uint4* __restrict__ x, int nvec, int k,
                         const int32_t* __restrict__ slot, const float* __restrict__ w,
                         uint4* __restrict__ recv_q, void* __restrict__ recv_s,
                         float* __restrict__ recv_w, int64_t sld)
{
    constexpr int kPass = 64 * VPT;
    __shared__ uint32_t srow[kPass / kLanesPerBlock];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* s = slot + t * k;
    const int32_t sl = token_slots(s, k);
    const int units = nvec >> 1;
    const int nb = nvec >> 4;

    if (recv_w != nullptr && tid < k && sl >= 0) recv_w[sl] = w[t * k + tid];

    const uint4* xr = x + t * nvec;
    for (int p0 = 0; p0 < units; p0 += kPass) {
        uint4 d[VPT][2];
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int unit = p0 + tid + u * 64;
            if (unit < units) {
                d[u][0] = xr[2 * unit];
                d[u][1] = xr[2 * unit + 1];
            } else {
                d[u][0] = make_uint4(0u, 0u, 0u, 0u);
                d[u][1] = d[u][0];
            }
        }
        uint4 q[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            uint32_t sb;
            q[u] = quantise16<FMT, SM>(d[u][0], d[u][1], sb);
            if ((tid & (kLanesPerBlock - 1)) == 0) srow[(tid + u * 64) / kLanesPerBlock] = sb;
        }
        __syncthreads();
        const int b0 = p0 / kLanesPerBlock;
        const int pass_blocks = min(kPass / kLanesPerBlock, nb - b0);
        const uint32_t my_scale = tid < pass_blocks ? srow[tid] : 0u;
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r < 0) continue;
            const __amdgpu_buffer_rsrc_t dq = buffer_rsrc(recv_q + (int64_t)r * units, units * 16);
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int unit = p0 + tid + u * 64;
                if (unit < units) store_row16(dq, unit * 16, q[u]);
            }
            if (tid < pass_blocks) {
                const int64_t at = sld == 0 ? (int64_t)r * nb + b0 + tid : (int64_t)(b0 + tid) * sld + r;
                if (SM == kScaleUe8m0)
                    static_cast<uint8_t*>(recv_s)[at] = (uint8_t)my_scale;
                else
                    static_cast<uint32_t*>(recv_s)[at] = my_scale;
            }
        }
        __syncthreads();
    }
}

// Tiled cast (rows of more than 64 units, row-major scales): workgroup b
// is (token t, tile p of NL units = NL/8 scale blocks, slot group g of up to
// CS slots), and all of a token's workgroups run back to back on one
// XCD, so the pieces of a token's scale rows that different tiles write
// meet in that XCD's L2.  Each lane casts one unit; the first lane of each
// 8-lane block stores the block's scale per destination.  At T=8192, hidden 7168, k=8 this took 122 us against 126 us
// for one wavefront per token; with tiles spread over the XCDs it took
// 127 us.  Column-major scales (each a separate 4-byte store) measured
// slower tiled, 163 us against 140 us, and keep one wavefront per token.
//
// Tiles are 128 lanes (NL = kTileLanes), or 64 where the last 128-lane tile
// would be at most half full (narrow_tiles: hidden 2176-3072, 5120, 7168,
// ...): hidden 3072 took 52.7 us in 64-lane tiles against 59.1 us in
// 128-lane ones, hidden 7168 1-2% less.  On rows of whole 128-lane tiles
// widths of 64 to 512 lanes measured within 3% of 128 (hidden 4096-16384,
// T=8192, k=8).
//
// Slot groups (CS slots per workgroup): 4 on rows of more than 256 units,
// 8 on shorter ones.  With groups of 4 each tile is cast once per group,
// and each workgroup stores 4 code pieces instead of 8.  Against groups of
// 8 (interleaved A/B rounds, T=8192, k=8, fp32 scales) groups of 4 ran
// 1.7-2.3% faster at hidden 7168, 2.6% at 8192 and 5.1% at 16384, within
// 1% at 4096, and 1-8% slower at hidden 1536-3072; with power-of-two and
// UE8M0 scales the two were within 0.2% at 7168.  Groups of 2 were 33%
// slower, and putting a tile's groups together on one XCD, or plain order,
// instead of a token's tiles, 3-5% slower.
constexpr int kCastSlotsLong = 4;
constexpr int kCastSlotsShort = 8;
constexpr int kCastLongUnits = 2 * kTileLanes;   // rows of more than this many units

// WS: instead of a scale row per destination, the token's scale row goes
// once (from slot group 0) to a per-token workspace [T, nb], for the
// column-major pass below.
template <int FMT, int SM, int NL, int CS, bool WS = false>
__global__ __launch_bounds__(NL)
void dispatch_fp8_tile_kernel(const uint4* __restrict__ x, int nvec, int k, int tpr, int64_t T,
                              int groups, const int32_t* __restrict__ slot,
                              const float* __restrict__ w, uint4* __restrict__ recv_q,
                              void* __restrict__ recv_s, float* __restrict__ recv_w)
{
    int64_t t;
    int within;
    if (!xcd_tile(blockIdx.x, tpr * groups, T, t, within)) return;
    const int p = within / groups;
    const int g = within - p * groups;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int units = nvec >> 1;
    const int nb = nvec >> 4;
    const int j0 = g * CS;
    const int32_t sl = lane < CS && j0 + lane < k ? slot[t * k + j0 + lane] : -1;
    if (recv_w != nullptr && p == 0 && tid < CS && sl >= 0) recv_w[sl] = w[t * k + j0 + tid];
    int32_t r[CS];
#pragma unroll
    for (int q = 0; q < CS; ++q) r[q] = lane_value(sl, q);

    // units past the row end (last tile) read zeros and store nothing; whole
    // blocks lie on one side of the row end (units is a multiple of 8)
    const int unit = p * NL + tid;
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + t * nvec, nvec * 16);
    const uint4 d0 = load_row16<0>(xs, unit * 32);
    const uint4 d1 = load_row16<0>(xs, unit * 32 + 16);
    uint32_t sb;
    const uint4 code = quantise16<FMT, SM>(d0, d1, sb);
    // every lane of a block holds the block's scale; the block's first lane
    // stores it, so lanes 0, 8, ..., 56 of a wavefront write its 8
    // consecutive scales (no exchange between lanes)
    const uint32_t my_scale = sb;
    const int bk = unit / kLanesPerBlock;
    const bool scale_lane = (lane & (kLanesPerBlock - 1)) == 0 && bk < nb;
    if (WS && g == 0 && scale_lane) {
        const int64_t at = t * nb + bk;
        if (SM == kScaleUe8m0)
            static_cast<uint8_t*>(recv_s)[at] = (uint8_t)my_scale;
        else
            static_cast<uint32_t*>(recv_s)[at] = my_scale;
    }
#pragma unroll
    for (int q = 0; q < CS; ++q) {
        if (r[q] < 0) continue;
        if (unit < units)
            store_row16(buffer_rsrc(recv_q + (int64_t)r[q] * units, units * 16), unit * 16, code);
        if (!WS && scale_lane) {
            const int64_t at = (int64_t)r[q] * nb + bk;
            if (SM == kScaleUe8m0)
                static_cast<uint8_t*>(recv_s)[at] = (uint8_t)my_scale;
            else
                static_cast<uint32_t*>(recv_s)[at] = my_scale;
        }
    }
}

// Column-major scales from the per-token workspace (DeepEP page, dispatch()
// use_tma_aligned_col_major_sf: each block's scales contiguous over rows).
// One lane per receive row r, so a wavefront writes 64 consecutive entries
// of a block's column at a time; written one row at a time, a row's scales
// would be nb separate 4-byte stores into nb lines.  t = src[r] is taken
// only if one of t's slots is r, so rows nothing maps to (padding, dropped
// pairs, rows past N) are skipped whatever src holds there.
//
// The pieces of a row (4 scales each when nb % 4 == 0: 16 bytes of fp32 or
// 4 UE8M0 bytes) are split over gridDim.y workgroups, part blockIdx.y taking
// pieces part, part + gridDim.y, ..., kColBatch of them loaded (clamped
// indices, no branch between the loads) before their stores.  The kernel is
// bound by its chain of dependent loads (src, then t's slot row, then the
// scale row) rather than by its stores (14.7 MB at T=8192, hidden 7168,
// k=8), so the slot row is read 16 bytes at a time when aligned (V4).
// Measured there (device time): 11.6 us with 8 pieces per batch over 4
// parts and 4-byte slot loads, 8.1 with 4 per batch and 16-byte slot loads,
// 7.7 with 4 per batch over 2 parts; 1 part, or 8 per batch, 7.9-8.6.
// Loading the first pieces together with the slot row, ahead of the check,
// measured slower (10.3 us).
constexpr int kColmajorParts = 2;   // workgroups per 256 rows
constexpr int kColBatch = 4;        // pieces loaded before their stores

template <int SM> struct ColPiece;          // 4 scales of one row
template <> struct ColPiece<kScaleFp32> {
    using V = uint4;
    __device__ static void put(void* out, int64_t at, int64_t ld, V v) {
        uint32_t* o = static_cast<uint32_t*>(out) + at;
        o[0] = v.x; o[ld] = v.y; o[2 * ld] = v.z; o[3 * ld] = v.w;
    }
};
template <> struct ColPiece<kScaleUe8m0> {
    using V = uint32_t;
    __device__ static void put(void* out, int64_t at, int64_t ld, V v) {
        uint8_t* o = static_cast<uint8_t*>(out) + at;
        o[0] = (uint8_t)v; o[ld] = (uint8_t)(v >> 8); o[2 * ld] = (uint8_t)(v >> 16);
        o[3 * ld] = (uint8_t)(v >> 24);
    }
};

// whether r is one of the k slots of the row at s (aligned to 16 bytes and
// k % 4 == 0 when V4); every load is issued before the first comparison
template <bool V4>
__device__ __forceinline__ bool row_is_slot(const int32_t* __restrict__ s, int k, int64_t r)
{
    bool mine = false;
    if (V4) {
        const int4* s4 = reinterpret_cast<const int4*>(s);
        const int n4 = k / 4;
        for (int j0 = 0; j0 < n4; j0 += 2) {
            int4 v[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) v[q] = s4[min(j0 + q, n4 - 1)];   // clamped: no branch
#pragma unroll
            for (int q = 0; q < 2; ++q)
                mine |= j0 + q < n4 && (v[q].x == r || v[q].y == r || v[q].z == r || v[q].w == r);
        }
    } else {
        for (int j0 = 0; j0 < k; j0 += 8) {
            int32_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = s[min(j0 + q, k - 1)];
#pragma unroll
            for (int q = 0; q < 8; ++q) mine |= j0 + q < k && v[q] == r;
        }
    }
    return mine;
}

template <int SM, bool V4>
__global__ __launch_bounds__(256)
void scales_colmajor_kernel(const void* __restrict__ ws, bool vec, const int32_t* __restrict__ src,
                            const int32_t* __restrict__ slot, int64_t T, int k, int nb,
                            int64_t rows, void* __restrict__ scales, int64_t ld)
{
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int part = blockIdx.y, parts = gridDim.y;
    if (r >= rows) return;
    const int32_t t = src[r];
    if (t < 0 || t >= T) return;
    if (!vec) {                // one scale at a time
        if (!row_is_slot<V4>(slot + (int64_t)t * k, k, r)) return;
        for (int b = part; b < nb; b += parts) {
            if (SM == kScaleUe8m0)
                static_cast<uint8_t*>(scales)[(int64_t)b * ld + r] =
                    static_cast<const uint8_t*>(ws)[(int64_t)t * nb + b];
            else
                static_cast<uint32_t*>(scales)[(int64_t)b * ld + r] =
                    static_cast<const uint32_t*>(ws)[(int64_t)t * nb + b];
        }
        return;
    }
    using P = ColPiece<SM>;
    using V = typename P::V;
    const V* in = reinterpret_cast<const V*>(static_cast<const uint8_t*>(ws) +
                                             (int64_t)t * nb * (SM == kScaleUe8m0 ? 1 : 4));
    const int np = nb / 4;
    if (!row_is_slot<V4>(slot + (int64_t)t * k, k, r)) return;
    for (int c0 = part; c0 < np; c0 += kColBatch * parts) {
        V v[kColBatch];
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) v[u] = in[min(c0 + u * parts, np - 1)];   // clamped
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) {
            const int c = c0 + u * parts;
            if (c < np) P::put(scales, (int64_t)4 * c * ld + r, ld, v[u]);
        }
    }
}

// Pre-quantized input (one wavefront per token; the cast's tiling, tried
// here too in both workgroup orders, measured 117 us against 114 us): the
// 8-bit code row (hidden bytes, VPT 16-byte units
// per lane per pass) and the fp32 scale row of token t are copied to every
// unmasked slot.  No arithmetic: any 8-bit float format passes through.
// Output scales row-major (sld == 0) or column-major [nb, sld].
//
// SG > 0: one wavefront per (token, group of SG slots) instead of per token,
// XCD-aware, for row-major scales on rows of more than 256 units: with
// groups of 4 the
// copy took 106.9 against 111.1 us at T=8192, hidden 7168, k=8 (interleaved
// A/B) and 62.6 against 63.5 us at 4096; at hidden 2048, and with
// column-major scales, groups were as fast or up to 11% slower.
// SCALES false: the code rows only (the two-pass column-major copy writes
// the scales in its second pass).
template <int VPT, int SG, bool SCALES>
__global__ __launch_bounds__(64)
void dispatch_prequant_kernel(const uint4* __restrict__ xq, const float* __restrict__ xs,
                              int units, int k, const int32_t* __restrict__ slot,
                              const float* __restrict__ w, uint4* __restrict__ recv_q,
                              float* __restrict__ recv_s, float* __restrict__ recv_w, int64_t sld,
                              int64_t num_tokens)
{
    constexpr int kPass = 64 * VPT;
    // grouped: a token's wavefronts run back to back on one XCD (xcd_tile),
    // so its code row comes from HBM once and then from that XCD's L2
    int64_t t = blockIdx.x;
    int gi = 0;
    if (SG > 0 && !xcd_tile(blockIdx.x, (k + SG - 1) / SG, num_tokens, t, gi)) return;
    const int j0 = gi * SG;
    const int kk = SG == 0 ? k : min(SG, k - j0);   // this wavefront's slots: j0 .. j0+kk-1
    const int tid = threadIdx.x;
    const int32_t sl = tid < kk ? slot[t * k + j0 + tid] : -1;
    const int nb = units >> 3;

    if (recv_w != nullptr && tid < kk && sl >= 0) recv_w[sl] = w[t * k + j0 + tid];

    const uint4* qr = xq + t * units;
    for (int p0 = 0; p0 < units; p0 += kPass) {
        uint4 d[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int unit = p0 + tid + u * 64;
            d[u] = unit < units ? qr[unit] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) keep(d[u]);
        for (int j = 0; j < kk; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r < 0) continue;
            const __amdgpu_buffer_rsrc_t dq = buffer_rsrc(recv_q + (int64_t)r * units, units * 16);
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int unit = p0 + tid + u * 64;
                if (unit < units) store_row16(dq, unit * 16, d[u]);
            }
        }
    }
    if (!SCALES) return;              // scales written by a later pass
    // the scale row: 64 floats per round
    for (int b0 = 0; b0 < nb; b0 += 64) {
        const int b = b0 + tid;
        const float v = b < nb ? xs[t * nb + b] : 0.0f;
        for (int j = 0; j < kk; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r >= 0 && b < nb) recv_s[sld == 0 ? (int64_t)r * nb + b : (int64_t)b * sld + r] = v;
        }
    }
}

struct Shape {
    int nt;
    int vpt;
};

// 64 lanes for rows of up to 64 vectors, else 128.  Vectors per lane: the
// largest VPT <= 8 with 128*VPT dividing the row, so the row is covered by
// whole passes (896 = 128*7 vectors for hidden 7168); for other rows the
// widest passes that fit, plus a one-vector-per-lane tail.
Shape pick_shape(int nvec)
{
    Shape s;
    if (nvec <= 64) {
        s.nt = 64;
        s.vpt = 1;
        return s;
    }
    s.nt = 128;
    const int fit = nvec / 128;
    s.vpt = fit < 1 ? 1 : (fit > 8 ? 8 : fit);
    for (int v = 8; v >= 1; --v) {
        if (nvec % (128 * v) == 0) {
            s.vpt = v;
            break;
        }
    }
    return s;
}

#define EP_DISPATCH_CASES(KERNEL, ...)                                                   \
    switch (sh.nt * 16 + sh.vpt) {                                                       \
    case 64 * 16 + 1: hipLaunchKernelGGL((KERNEL<64, 1>), grid, dim3(64), 0, stream, __VA_ARGS__); break;   \
    case 128 * 16 + 1: hipLaunchKernelGGL((KERNEL<128, 1>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 2: hipLaunchKernelGGL((KERNEL<128, 2>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 3: hipLaunchKernelGGL((KERNEL<128, 3>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 4: hipLaunchKernelGGL((KERNEL<128, 4>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 5: hipLaunchKernelGGL((KERNEL<128, 5>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 6: hipLaunchKernelGGL((KERNEL<128, 6>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    case 128 * 16 + 7: hipLaunchKernelGGL((KERNEL<128, 7>), grid, dim3(128), 0, stream, __VA_ARGS__); break; \
    default: hipLaunchKernelGGL((KERNEL<128, 8>), grid, dim3(128), 0, stream, __VA_ARGS__); break;           \
    }

}  // namespace

hipError_t launch_dispatch_bf16(const void* x, int64_t num_tokens, int hidden, int num_topk,
                                const int32_t* slot, const float* topk_weights, void* recv_x,
                                float* recv_weights, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    // rows of 257-511 vectors whose last 128-lane tile would be at most half
    // full go in 64-lane tiles: at T=8192, k=8 (interleaved A/B) hidden
    // 2560, 3200 and 3584 took 74.1, 93.0 and 103.5 us against 80.3, 98.6
    // and 111.9 us for one workgroup per token, and 2-5% less at T=4096 or
    // k=4; at 129-192 vectors (hidden 1152-1536) they were 3% faster to 7%
    // slower, and those rows stay per token
    const bool narrow = nvec > 2 * kTileLanes && nvec < kMinTiledDispatchVectors && narrow_tiles(nvec);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (nvec + lanes - 1) / lanes;
    const int groups = (num_topk + kSlotsPerGroup - 1) / kSlotsPerGroup;
    const int64_t num_tiles = num_tokens * tpr;
    const int64_t blocks = (num_tiles + 7) / 8 * 8 * groups;
    if ((narrow || tile_dispatch(nvec, num_tokens * num_topk)) && blocks <= INT32_MAX) {
        if (narrow)
            hipLaunchKernelGGL(dispatch_bf16_tile_kernel<kTileLanes / 2>, dim3((unsigned)blocks),
                               dim3(kTileLanes / 2), 0, stream, static_cast<const uint4*>(x), nvec,
                               num_topk, tpr, num_tiles, groups, slot, topk_weights,
                               static_cast<uint4*>(recv_x), recv_weights);
        else
            hipLaunchKernelGGL(dispatch_bf16_tile_kernel<kTileLanes>, dim3((unsigned)blocks),
                               dim3(kTileLanes), 0, stream, static_cast<const uint4*>(x), nvec,
                               num_topk, tpr, num_tiles, groups, slot, topk_weights,
                               static_cast<uint4*>(recv_x), recv_weights);
        return hipGetLastError();
    }
    const Shape sh = pick_shape(nvec);
    const dim3 grid((unsigned)num_tokens);
    EP_DISPATCH_CASES(dispatch_bf16_kernel, static_cast<const uint4*>(x), nvec, num_topk, slot,
                      topk_weights, static_cast<uint4*>(recv_x), recv_weights)
    return hipGetLastError();
}

// the largest VPT <= 8 with 64*VPT dividing the row's units (448 = 64*7 at
// hidden 7168), else the widest that fits
static int units_per_lane(int units)
{
    const int fit = units / 64;
    int vpt = fit < 1 ? 1 : (fit > 8 ? 8 : fit);
    for (int v = 8; v >= 1; --v) {
        if (units % (64 * v) == 0) {
            vpt = v;
            break;
        }
    }
    return vpt;
}

template <int FMT, int SM>
static void launch_fp8_shape(int vpt, dim3 grid, hipStream_t stream, const uint4* xx, int nvec,
                             int k, const int32_t* slot, const float* w, uint4* qq, void* ss,
                             float* rw, int64_t sld)
{
#define EP_FP8(V)                                                                             \
    hipLaunchKernelGGL((dispatch_fp8_kernel<V, FMT, SM>), grid, dim3(64), 0, stream, xx, nvec, \
                       k, slot, w, qq, ss, rw, sld)
    switch (vpt) {
    case 1: EP_FP8(1); break;
    case 2: EP_FP8(2); break;
    case 3: EP_FP8(3); break;
    case 4: EP_FP8(4); break;
    case 5: EP_FP8(5); break;
    case 6: EP_FP8(6); break;
    case 7: EP_FP8(7); break;
    default: EP_FP8(8); break;
    }
#undef EP_FP8
}

hipError_t launch_dispatch_fp8(const void* x, int64_t num_tokens, int hidden, int num_topk,
                               const int32_t* slot, const float* topk_weights, int format,
                               int scale_mode, void* recv_q, void* recv_scales,
                               float* recv_weights, int64_t scale_ld, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const int vpt = units_per_lane(hidden / 16);
    const dim3 grid((unsigned)num_tokens);
    const uint4* xx = static_cast<const uint4*>(x);
    uint4* qq = static_cast<uint4*>(recv_q);
    const int units = hidden / 16;
    const bool narrow = narrow_tiles(units);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (units + lanes - 1) / lanes;
    const int cs = units > kCastLongUnits ? kCastSlotsLong : kCastSlotsShort;
    const int groups = (num_topk + cs - 1) / cs;
    const int64_t blocks = (num_tokens + 7) / 8 * 8 * tpr * groups;
    const bool tiled = units > 64 && blocks <= INT32_MAX && scale_ld == 0;
#define EP_FP8_LAUNCH(F, M, NL, CS)                                                          \
    hipLaunchKernelGGL((dispatch_fp8_tile_kernel<F, M, NL, CS>), dim3((unsigned)blocks), dim3(NL), \
                       0, stream, xx, nvec, num_topk, tpr, num_tokens, groups, slot, topk_weights, \
                       qq, recv_scales, recv_weights)
#define EP_FP8_TILES(F, M, NL)                                                                \
    {                                                                                         \
        if (cs == kCastSlotsLong)                                                             \
            EP_FP8_LAUNCH(F, M, NL, kCastSlotsLong);                                          \
        else                                                                                  \
            EP_FP8_LAUNCH(F, M, NL, kCastSlotsShort);                                         \
    }
#define EP_FP8_MODE(F, M)                                                                    \
    if (tiled && narrow)                                                                     \
        EP_FP8_TILES(F, M, kTileLanes / 2)                                                   \
    else if (tiled)                                                                          \
        EP_FP8_TILES(F, M, kTileLanes)                                                       \
    else                                                                                     \
        launch_fp8_shape<F, M>(vpt, grid, stream, xx, nvec, num_topk, slot, topk_weights, qq, \
                               recv_scales, recv_weights, scale_ld)
    if (format == kE5M2) {
        if (scale_mode == kScalePow2) EP_FP8_MODE(kE5M2, kScalePow2);
        else if (scale_mode == kScaleUe8m0) EP_FP8_MODE(kE5M2, kScaleUe8m0);
        else EP_FP8_MODE(kE5M2, kScaleFp32);
    } else {
        if (scale_mode == kScalePow2) EP_FP8_MODE(kE4M3, kScalePow2);
        else if (scale_mode == kScaleUe8m0) EP_FP8_MODE(kE4M3, kScaleUe8m0);
        else EP_FP8_MODE(kE4M3, kScaleFp32);
    }
#undef EP_FP8_MODE
#undef EP_FP8_TILES
#undef EP_FP8_LAUNCH
    return hipGetLastError();
}


size_t colmajor_workspace_bytes(int64_t num_tokens, int hidden, int scale_mode)
{
    const size_t bytes = (size_t)num_tokens * (hidden / 128) * (scale_mode == kScaleUe8m0 ? 1 : 4);
    return (bytes + 255) & ~(size_t)255;
}

// The column pass: rows [0, rows) of [nb, scale_ld] scales from per-token
// scale rows ws [T, nb] (fp32, or bytes for UE8M0); vec: nb % 4 == 0 and
// ws 16-byte aligned, so each row is read in pieces of 4 scales.
static hipError_t launch_scales_colmajor(const void* ws, bool vec, const int32_t* src,
                                         const int32_t* slot, int64_t num_tokens, int num_topk,
                                         int nb, int scale_mode, int64_t rows, void* recv_scales,
                                         int64_t scale_ld, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    const int pieces = vec ? nb / 4 : nb;
    const dim3 grid((unsigned)((rows + 255) / 256), (unsigned)std::min(kColmajorParts, pieces));
    const bool v4 = num_topk % 4 == 0 && (reinterpret_cast<uintptr_t>(slot) & 15) == 0;
#define EP_CM_COLS(SM, V4)                                                                      \
    hipLaunchKernelGGL((scales_colmajor_kernel<SM, V4>), grid, dim3(256), 0, stream, ws, vec, src, \
                       slot, num_tokens, num_topk, nb, rows, recv_scales, scale_ld)
    if (scale_mode == kScaleUe8m0) {
        if (v4) EP_CM_COLS(kScaleUe8m0, true);
        else EP_CM_COLS(kScaleUe8m0, false);
    } else {
        if (v4) EP_CM_COLS(kScaleFp32, true);
        else EP_CM_COLS(kScaleFp32, false);
    }
#undef EP_CM_COLS
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8_colmajor(const void* x, int64_t num_tokens, int hidden,
                                        int num_topk, const int32_t* slot, const int32_t* src,
                                        const float* topk_weights, int format, int scale_mode,
                                        void* recv_q, void* recv_scales, float* recv_weights,
                                        int64_t scale_ld, int64_t rows, void* workspace,
                                        hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const int units = hidden / 16;
    const int nb = hidden / 128;
    const bool narrow = narrow_tiles(units);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (units + lanes - 1) / lanes;
    const int cs = units > kCastLongUnits ? kCastSlotsLong : kCastSlotsShort;
    const int groups = (num_topk + cs - 1) / cs;
    const int64_t blocks = (num_tokens + 7) / 8 * 8 * tpr * groups;
    if (units <= 64 || blocks > INT32_MAX)   // short rows: the one-wavefront-per-token cast
        return launch_dispatch_fp8(x, num_tokens, hidden, num_topk, slot, topk_weights, format,
                                   scale_mode, recv_q, recv_scales, recv_weights, scale_ld, stream);
    const uint4* xx = static_cast<const uint4*>(x);
    uint4* qq = static_cast<uint4*>(recv_q);
#define EP_CM_LAUNCH(F, M, NL, CS)                                                              \
    hipLaunchKernelGGL((dispatch_fp8_tile_kernel<F, M, NL, CS, true>), dim3((unsigned)blocks),     \
                       dim3(NL), 0, stream, xx, nvec, num_topk, tpr, num_tokens, groups, slot,    \
                       topk_weights, qq, workspace, recv_weights)
#define EP_CM_TILES(F, M)                                                                       \
    {                                                                                           \
        if (narrow && cs == kCastSlotsLong) EP_CM_LAUNCH(F, M, kTileLanes / 2, kCastSlotsLong);   \
        else if (narrow) EP_CM_LAUNCH(F, M, kTileLanes / 2, kCastSlotsShort);                    \
        else if (cs == kCastSlotsLong) EP_CM_LAUNCH(F, M, kTileLanes, kCastSlotsLong);           \
        else EP_CM_LAUNCH(F, M, kTileLanes, kCastSlotsShort);                                    \
    }
    if (format == kE5M2) {
        if (scale_mode == kScalePow2) EP_CM_TILES(kE5M2, kScalePow2)
        else if (scale_mode == kScaleUe8m0) EP_CM_TILES(kE5M2, kScaleUe8m0)
        else EP_CM_TILES(kE5M2, kScaleFp32)
    } else {
        if (scale_mode == kScalePow2) EP_CM_TILES(kE4M3, kScalePow2)
        else if (scale_mode == kScaleUe8m0) EP_CM_TILES(kE4M3, kScaleUe8m0)
        else EP_CM_TILES(kE4M3, kScaleFp32)
    }
#undef EP_CM_TILES
#undef EP_CM_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || rows == 0) return err;
    return launch_scales_colmajor(workspace, (nb & 3) == 0, src, slot, num_tokens, num_topk, nb,
                                  scale_mode, rows, recv_scales, scale_ld, stream);
}

constexpr int kPrequantSlots = 4;          // slots per wavefront when grouped
constexpr int kPrequantGroupUnits = 256;    // grouped for rows of more than this many units

hipError_t launch_dispatch_prequant(const void* xq, const float* xs, int64_t num_tokens,
                                    int hidden, int num_topk, const int32_t* slot,
                                    const float* topk_weights, void* recv_q, float* recv_scales,
                                    float* recv_weights, int64_t scale_ld, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int units = hidden / 16;
    const int vpt = units_per_lane(units);
    const dim3 grid((unsigned)num_tokens);
    const uint4* qq = static_cast<const uint4*>(xq);
    uint4* rq = static_cast<uint4*>(recv_q);

    const int64_t gblocks = (num_tokens + 7) / 8 * 8 * ((num_topk + kPrequantSlots - 1) / kPrequantSlots);
    const bool grouped = scale_ld == 0 && units > kPrequantGroupUnits && gblocks <= INT32_MAX;
    const dim3 ggrid((unsigned)gblocks);
#define EP_PQ_SC(V, SC)                                                                          \
    if (grouped)                                                                               \
        hipLaunchKernelGGL((dispatch_prequant_kernel<V, kPrequantSlots, SC>), ggrid, dim3(64), 0, \
                           stream, qq, xs, units, num_topk, slot, topk_weights, rq, recv_scales,   \
                           recv_weights, scale_ld, num_tokens);                                   \
    else                                                                                       \
        hipLaunchKernelGGL((dispatch_prequant_kernel<V, 0, SC>), grid, dim3(64), 0, stream, qq,    \
                           xs, units, num_topk, slot, topk_weights, rq, recv_scales, recv_weights, \
                           scale_ld, num_tokens)
#define EP_PQ(V)                                                                                   \
    if (recv_scales != nullptr) { EP_PQ_SC(V, true); } else { EP_PQ_SC(V, false); }
    switch (vpt) {
    case 1: EP_PQ(1); break;
    case 2: EP_PQ(2); break;
    case 3: EP_PQ(3); break;
    case 4: EP_PQ(4); break;
    case 5: EP_PQ(5); break;
    case 6: EP_PQ(6); break;
    case 7: EP_PQ(7); break;
    default: EP_PQ(8); break;
    }
#undef EP_PQ
#undef EP_PQ_SC
    return hipGetLastError();
}

// Pre-quantized rows with column-major scales in two passes: the code rows
// as in the row-major copy (a token's wavefronts on one XCD), then the
// column pass reading each receive row's scales straight from x_scales,
// which already holds every token's scale row once.
hipError_t launch_dispatch_prequant_colmajor(const void* xq, const float* xs, int64_t num_tokens,
                                             int hidden, int num_topk, const int32_t* slot,
                                             const int32_t* src, const float* topk_weights,
                                             void* recv_q, float* recv_scales, float* recv_weights,
                                             int64_t scale_ld, int64_t rows, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    hipError_t err = launch_dispatch_prequant(xq, xs, num_tokens, hidden, num_topk, slot,
                                              topk_weights, recv_q, nullptr, recv_weights, 0, stream);
    if (err != hipSuccess) return err;
    const int nb = hidden / 128;
    const bool vec = (nb & 3) == 0 && (reinterpret_cast<uintptr_t>(xs) & 15) == 0;
    return launch_scales_colmajor(xs, vec, src, slot, num_tokens, num_topk, nb, kScaleFp32, rows,
                                  recv_scales, scale_ld, stream);
}

}  // namespace ep

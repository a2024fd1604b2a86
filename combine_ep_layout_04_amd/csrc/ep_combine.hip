// ep_combine.hip -- weighted reduction of expert-output rows back into
// token order.
//
// Passages: NCCL EP page, nccl_ep.cc, ncclEpCombine (low-latency branch:
// bf16 expert outputs reduced to [T, hidden] bf16 with topk_weights [T, k]
// fp32; high-throughput forward combine carries tokens only, i.e. unit
// weights); DeepEP page, combine().
//
//   out[t] = bf16_rne( sum_{j = 0..k-1, slot[t,j] >= 0} w[t,j] * y[slot[t,j]] )
//
// accumulated in fp32, one fused multiply-add per term, in increasing j,
// starting from +0; the bf16 rounding is done once at the end.
//
// Design (HBM-bound): one workgroup per (token, 2 KiB tile of the row),
// one 16-byte column vector per lane.  The lane loads its vector from the
// k source rows back to back (k independent loads in flight before the
// first is consumed), reduces them in j order and stores the result once,
// as a streaming store.  Each loaded byte is used once by the lane that
// loaded it, so the gather goes straight to registers; an LDS round trip
// would add traffic without reuse.  The loads carry the non-temporal hint:
// the expert outputs are read exactly once, and streaming them past the
// caches measured ~12% faster than cached loads on MI355X.  k is a template
// parameter for k <= 8 so the loads are fully unrolled.
//
// The output goes out with streaming stores too.  Plain stores leave the
// output's write-back to whatever runs next: at T=8192, hidden 7168, k=8
// the combine then reads 188 us in its own events but 202 us once a
// following read pass is charged for the write-back; the tiled kernel with
// streaming stores takes 185 us either way.  Tiles are 128 lanes, or 64
// where the last 128-lane tile would be at most half full (narrow_tiles:
// hidden 1032-1536, 2560, 3584, ...): hidden 1152, 1280, 1536 and 3584
// took 33.3, 36.2, 42.1 and 93.3 us in 64-lane tiles against 37.7, 40.4,
// 45.3 and 96.7 us (T=8192, k=8).  Rows of at most 64 vectors, and grids past 2^31
// workgroups, keep one workgroup per token.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 round-to-nearest-even on the bit pattern (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void fma8(float (&acc)[8], float wt, const uint4& d)
{
    acc[0] = __builtin_fmaf(wt, bf16_lo(d.x), acc[0]);
    acc[1] = __builtin_fmaf(wt, bf16_hi(d.x), acc[1]);
    acc[2] = __builtin_fmaf(wt, bf16_lo(d.y), acc[2]);
    acc[3] = __builtin_fmaf(wt, bf16_hi(d.y), acc[3]);
    acc[4] = __builtin_fmaf(wt, bf16_lo(d.z), acc[4]);
    acc[5] = __builtin_fmaf(wt, bf16_hi(d.z), acc[5]);
    acc[6] = __builtin_fmaf(wt, bf16_lo(d.w), acc[6]);
    acc[7] = __builtin_fmaf(wt, bf16_hi(d.w), acc[7]);
}

__device__ __forceinline__ uint4 pack8(const float (&acc)[8])
{
    uint4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    return o;
}

// Buffer resource over one expert-output row: a masked slot gets a
// resource of zero bytes, so its loads return zeros without touching
// memory and the load sequence needs no branch.  (Raw buffer, stride 0,
// 32-bit data format word of the gfx9 resource descriptor.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint4* y, int32_t r, int nvec)
{
    const uint4* base = y + (int64_t)(r < 0 ? 0 : r) * nvec;
    const int bytes = r < 0 ? 0 : nvec * 16;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(base), (short)0, bytes, 0x00020000);
}

// Cache-policy bits of a gfx950 buffer instruction: bit 1 is "nt"
// (non-temporal, streaming).
constexpr int kLoadNT = 2;

// 16 bytes at vector v of the resource; past the resource's end it reads 0.
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int v)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, kLoadNT));
}

// K > 0: exactly K = k slots, unrolled, U column vectors per lane per
// iteration.  K == 0: any k (runtime loop, one vector per iteration).
// Lane j of every wavefront holds slot[t, j] and w[t, j] (k <= 64); they are
// read back as wavefront-uniform values with readlane.
//
// row_w / out_w (both or neither): the backward of dispatch also gathers the
// per-row weight gradients back to the pairs, out_w[t, j] = row_w[slot[t, j]]
// (0 for a masked pair).
template <int NT, int U, int K>
__global__ __launch_bounds__(NT)
void combine_kernel(const uint4* __restrict__ y, const int32_t* __restrict__ slot,
                    const float* __restrict__ w, int nvec, int k, uint4* __restrict__ out,
                    const float* __restrict__ row_w, float* __restrict__ out_w)
{
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kk = K > 0 ? K : k;
    const int32_t sl = lane < kk ? slot[t * kk + lane] : -1;
    const float wl = lane < kk ? (w ? w[t * kk + lane] : 1.0f) : 0.0f;
    const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(out + t * nvec, nvec * 16);
    if (out_w != nullptr && tid < kk) out_w[t * kk + tid] = sl >= 0 ? row_w[sl] : 0.0f;

    if constexpr (K > 0) {
        // A masked slot reads zeros through an empty resource and gets
        // weight 0, so its term fma(0, 0, acc) leaves acc's value unchanged
        // (at most an accumulated -0 turns into +0) and no branch is needed.
        // Vectors past the row end also read zeros and are not stored.
        __amdgpu_buffer_rsrc_t rs[K];
        float g[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(sl, j);
            rs[j] = row_rsrc(y, r, nvec);
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
            g[j] = r >= 0 ? wj : 0.0f;
        }
        for (int v0 = tid; v0 < nvec; v0 += NT * U) {
            uint4 d[U][K];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < K; ++j) d[u][j] = load16(rs[j], v0 + u * NT);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < K; ++j) fma8(acc, g[j], d[u][j]);
                if (v0 + u * NT < nvec) store_row16(ors, (v0 + u * NT) * 16, pack8(acc));
            }
        }
    } else {
        // the trip count is the same for every lane, so readlane always runs
        // with the whole wavefront active (it reads other lanes' registers,
        // whose values are only kept for lanes that are active); past the
        // row end the loads read 0 and nothing is stored
        for (int v0 = 0; v0 < nvec; v0 += NT) {
            const int v = v0 + tid;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < kk; ++j) {
                const int32_t r = __builtin_amdgcn_readlane(sl, j);
                if (r < 0) continue;
                const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
                fma8(acc, g, load16(row_rsrc(y, r, nvec), v));
            }
            if (v < nvec) store_row16(ors, v * 16, pack8(acc));
        }
    }
}

// Tiled form: workgroup b is tile b % tpr (NL vectors) of token b / tpr.
// K > 0: exactly K = k slots, unrolled; K == 0: any k, 8 slots' loads in
// flight at a time (slots past k count as masked: zero data, zero weight).
template <int K, int NL>
__global__ __launch_bounds__(NL)
void combine_tile_kernel(const uint4* __restrict__ y, const int32_t* __restrict__ slot,
                         const float* __restrict__ w, int nvec, int k, int tpr,
                         uint4* __restrict__ out, const float* __restrict__ row_w,
                         float* __restrict__ out_w)
{
    const int64_t tile = blockIdx.x;
    const int64_t t = tile / tpr;
    const int p = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kk = K > 0 ? K : k;
    const int32_t sl = lane < kk ? slot[t * kk + lane] : -1;
    const float wl = lane < kk ? (w ? w[t * kk + lane] : 1.0f) : 0.0f;
    if (out_w != nullptr && p == 0 && tid < kk) out_w[t * kk + tid] = sl >= 0 ? row_w[sl] : 0.0f;

    const int v = p * NL + tid;             // past the row end: reads 0, stores nothing
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int kBatch = K > 0 ? K : 8;
    for (int j0 = 0; j0 < kk; j0 += kBatch) {
        uint4 d[kBatch];
        float g[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int j = j0 + q;
            const int32_t r = j < kk ? __builtin_amdgcn_readlane(sl, j) : -1;
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j & 63));
            g[q] = r >= 0 ? wj : 0.0f;
            d[q] = load16(row_rsrc(y, r, nvec), v);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) fma8(acc, g[q], d[q]);
    }
    if (v < nvec) store_row16(buffer_rsrc(out + t * nvec, nvec * 16), v * 16, pack8(acc));
}

template <int NT, int U>
void launch_shape(dim3 grid, hipStream_t stream, const uint4* y, const int32_t* slot,
                  const float* w, int nvec, int k, uint4* out, const float* row_w, float* out_w)
{
#define EP_COMBINE_K(KV)                                                                       \
    hipLaunchKernelGGL((combine_kernel<NT, U, KV>), grid, dim3(NT), 0, stream, y, slot, w, nvec, \
                       k, out, row_w, out_w)
    switch (k) {
    case 1: EP_COMBINE_K(1); break;
    case 2: EP_COMBINE_K(2); break;
    case 3: EP_COMBINE_K(3); break;
    case 4: EP_COMBINE_K(4); break;
    case 5: EP_COMBINE_K(5); break;
    case 6: EP_COMBINE_K(6); break;
    case 7: EP_COMBINE_K(7); break;
    case 8: EP_COMBINE_K(8); break;
    default: EP_COMBINE_K(0); break;
    }
#undef EP_COMBINE_K
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* slot, const float* topk_weights,
                          int64_t num_tokens, int hidden, int num_topk, void* out,
                          const float* row_w, float* out_w, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const dim3 grid((unsigned)num_tokens);
    const uint4* yy = static_cast<const uint4*>(y);
    uint4* oo = static_cast<uint4*>(out);
    const bool narrow = narrow_tiles(nvec);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (nvec + lanes - 1) / lanes;
    const int64_t tiles = num_tokens * tpr;
    if (nvec > 64 && tiles <= INT32_MAX) {
        const dim3 tg((unsigned)tiles);
#define EP_COMBINE_TILE_NL(KV, NL)                                                            \
    hipLaunchKernelGGL((combine_tile_kernel<KV, NL>), tg, dim3(NL), 0, stream, yy, slot,        \
                       topk_weights, nvec, num_topk, tpr, oo, row_w, out_w)
#define EP_COMBINE_TILE(KV)                                                                     \
    if (narrow)                                                                                 \
        EP_COMBINE_TILE_NL(KV, kTileLanes / 2);                                                 \
    else                                                                                        \
        EP_COMBINE_TILE_NL(KV, kTileLanes)
        switch (num_topk) {
        case 1: EP_COMBINE_TILE(1); break;
        case 2: EP_COMBINE_TILE(2); break;
        case 3: EP_COMBINE_TILE(3); break;
        case 4: EP_COMBINE_TILE(4); break;
        case 5: EP_COMBINE_TILE(5); break;
        case 6: EP_COMBINE_TILE(6); break;
        case 7: EP_COMBINE_TILE(7); break;
        case 8: EP_COMBINE_TILE(8); break;
        default: EP_COMBINE_TILE(0); break;
        }
#undef EP_COMBINE_TILE
#undef EP_COMBINE_TILE_NL
        return hipGetLastError();
    }
    // 256 lanes x 2 vectors for long rows (hidden >= 4096: 896 vectors at
    // 7168 take two iterations); smaller workgroups for short rows
    if (nvec <= 64)
        launch_shape<64, 1>(grid, stream, yy, slot, topk_weights, nvec, num_topk, oo, row_w, out_w);
    else if (nvec < 512)
        launch_shape<128, 2>(grid, stream, yy, slot, topk_weights, nvec, num_topk, oo, row_w, out_w);
    else
        launch_shape<256, 2>(grid, stream, yy, slot, topk_weights, nvec, num_topk, oo, row_w, out_w);
    return hipGetLastError();
}

}  // namespace ep

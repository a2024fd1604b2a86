// ep_backward.hip -- backward of the weighted combine.
//
// Passages: DeepEP page, "MoE Dispatch and Combine for Training/Inference
// with ElasticBuffer" (the backward of combine is a dispatch, the backward of
// dispatch is a combine that also returns the reduced weight gradients);
// NeMo fused_a2a page, HybridEPCombine.backward (redispatch the combined-
// output gradients through the saved layout); NCCL EP page, ncclEpCombine
// high-throughput branch (backward combine carries tokens and topk weight
// gradients).
//
// With out[t] = sum_j w[t,j] * y[slot[t,j]] and upstream gradient g [T, H]:
//   grad_y[slot[t,j]] = bf16( w[t,j] * g[t] )       one rounding of the exact
//                                                   product
//   grad_w[t,j]       = sum_c g[t,c] * y[slot[t,j], c]   fp32 accumulation
//
// Design (HBM-bound).  Rows that the bf16 dispatch tiles (tile_dispatch) go
// through two launches:
//   1. grad_y, tiled exactly like the bf16 dispatch: a 128-lane workgroup
//      per (token, 2 KiB tile, group of 4 slots), XCD-aware, loads its
//      vector of g[t] and stores bf16(w * g) to each slot's row;
//   2. grad_w (when wanted): one workgroup per token reads g[t] and streams
//      each y[slot] with fp32 dot products, storing nothing else.
// Each is one pattern HBM runs well: a write stream with few reads, and a
// read stream.  One fused pass moves fewer bytes (g is read once) but mixes
// reads and writes half and half; at T=8192, hidden 7168, k=8 it took
// 406.5 us against 359.1 us for the two launches (grad_y alone 221.0
// against 204.4 us), and at hidden 2048-4096 the split was 3-8% faster.
// Shorter rows keep the fused pass (hidden 1536: 97.2 fused against
// 106.5 us split).  Both forms give the same bits: the dot products are
// accumulated in the same order.
//
// The fused pass and the grad_w pass: one 128-lane workgroup per token
// reads g[t] once into registers (VPT 16-byte vectors per lane).  For each
// slot it streams the expert row y[slot] (when grad_w is wanted),
// accumulates the per-lane dot product with fp32 FMAs and (fused) writes the
// scaled gradient row with streaming 16-byte stores; the per-slot partial
// dots are reduced across the workgroup at the end (8 slots at a time).  The bf16 rounding of
// w * g uses the exact product error e = fma(w, g, -p) of p = fl32(w * g):
// p is on the same side of every bf16 rounding boundary as the exact product
// unless p is itself a boundary (a bf16 midpoint), where the sign of e
// decides; this is exact whenever |w * g| >= 2^-117.  The branch-free form
// of that rule measured ~1.6x faster than a branchy one.  A vector that may
// hold a smaller nonzero or a NaN product (found from the vector's smallest
// nonzero and largest |g|, once per vector, and the slot's weight) is
// rounded exactly in fp64 instead.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// bf16 round-to-nearest-even of the exact product w * g, branch-free.
// (p + 0x7FFF + c) >> 16 rounds p's bits; the carry-in c only matters when
// the low 16 bits of p are exactly 0x8000 (a bf16 midpoint), and there the
// exact product lies above the midpoint's magnitude iff e has p's sign, is
// on it iff e == 0 (then ties go to even: c = lsb).  So c is chosen without
// testing for the midpoint at all.
//
// e is exact when w = Mw 2^a, g = Mg 2^b (Mw < 2^24, Mg < 2^8 integers)
// have a + b >= -149: e is a multiple of 2^(a+b) below half an ulp of p.
// The exact product is below 2^(a+b+32), so |w g| >= 2^-117 guarantees it.
// Smaller nonzero products (where e may round to 0 and lose the side of a
// midpoint: w = 1.25 * 2^-32 + 2^-55, g = 2^-100 is one) and NaN products
// are left to bf16_of_product_exact; vector_needs_exact finds them.
__device__ __forceinline__ uint32_t bf16_of_product(float w, float g)
{
    const float p = w * g;
    const float e = __builtin_fmaf(w, g, -p);
    const uint32_t u = __float_as_uint(p);
    const uint32_t lsb = (u >> 16) & 1u;
    const uint32_t same_sign = (~(__float_as_uint(e) ^ u)) >> 31;
    const uint32_t c = e != 0.0f ? same_sign : lsb;
    return (u + 0x7FFFu + c) >> 16;
}

// The same rounding without the fast path's limits: the product is formed
// in fp64, where it is exact (at most 24 + 8 significant bits, exponent
// from -282 up), then rounded to nearest even on the bf16 grid: multiples
// of 2^-133 below 2^-126, otherwise 8 significant bits by an integer RNE on
// the fp64 bit pattern, where a result past the largest finite bf16 (an
// infinite product included) is infinity.  A NaN product gives the
// canonical quiet NaN 0x7FC0 (the sign and payload of a NaN a multiply
// makes are not portable).
__device__ __forceinline__ uint32_t bf16_of_product_exact(float w, float g)
{
    const double d = (double)w * (double)g;
    if (d != d) return 0x7FC0u;
    const uint64_t u = (uint64_t)__double_as_longlong(d);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a < 0x3810000000000000ull)   // |d| < 2^-126
        return sign | (uint32_t)__builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
    const uint64_t r = ((a + ((1ull << 44) - 1) + ((a >> 45) & 1ull)) >> 45) - ((uint64_t)(1023 - 127) << 7);
    return sign | (uint32_t)(r < 0x7F80ull ? r : 0x7F80ull);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// What one vector of 8 bf16 gradients contributes to that test, computed
// once and shared by every slot the vector is scaled for: `gmin`, the
// smallest nonzero |g| as fp32 (+inf past the bf16 range when all are 0),
// and whether any |g| is infinite or NaN.  Packed 16-bit operations on the
// bf16 magnitudes: m - 1 wraps 0 to 0xFFFF, so the minimum skips zeros.
struct GradStat {
    float gmin;
    bool special;
};

__device__ __forceinline__ GradStat grad_stat(const uint4& g)
{
    const u16x2 one = {1, 1};
    const u16x2 m0 = __builtin_bit_cast(u16x2, g.x & 0x7FFF7FFFu);
    const u16x2 m1 = __builtin_bit_cast(u16x2, g.y & 0x7FFF7FFFu);
    const u16x2 m2 = __builtin_bit_cast(u16x2, g.z & 0x7FFF7FFFu);
    const u16x2 m3 = __builtin_bit_cast(u16x2, g.w & 0x7FFF7FFFu);
    const u16x2 lo = __builtin_elementwise_min(__builtin_elementwise_min(m0 - one, m1 - one),
                                               __builtin_elementwise_min(m2 - one, m3 - one));
    const u16x2 hi = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                               __builtin_elementwise_max(m2, m3));
    const uint32_t mn = (uint32_t)min(lo.x, lo.y) + 1u;   // 0x10000 if all are 0
    GradStat st;
    st.gmin = __uint_as_float(min(mn, 0x7F80u) << 16);     // all 0: +inf
    st.special = max(hi.x, hi.y) >= 0x7F80u;
    return st;
}

// True when some product w * g of the vector may fall outside the fast
// path: a NaN or infinite w, an infinite or NaN g, or a nonzero product
// below 2^-116 (fl32(|w| gmin) is at most 2^-117 whenever the smallest
// exact nonzero product is, since rounding is monotone).
__device__ __forceinline__ bool vector_needs_exact(float w, const GradStat& st)
{
    return !(fabsf(w) <= 0x1.fffffep127f) || st.special || fabsf(w) * st.gmin < 0x1p-116f;
}

__device__ __forceinline__ uint4 scale_row8(float w, const uint4& g, const GradStat& st)
{
    uint4 o;
    if (!vector_needs_exact(w, st)) {
        o.x = bf16_of_product(w, bf16_lo(g.x)) | (bf16_of_product(w, bf16_hi(g.x)) << 16);
        o.y = bf16_of_product(w, bf16_lo(g.y)) | (bf16_of_product(w, bf16_hi(g.y)) << 16);
        o.z = bf16_of_product(w, bf16_lo(g.z)) | (bf16_of_product(w, bf16_hi(g.z)) << 16);
        o.w = bf16_of_product(w, bf16_lo(g.w)) | (bf16_of_product(w, bf16_hi(g.w)) << 16);
    } else {
        o.x = bf16_of_product_exact(w, bf16_lo(g.x)) | (bf16_of_product_exact(w, bf16_hi(g.x)) << 16);
        o.y = bf16_of_product_exact(w, bf16_lo(g.y)) | (bf16_of_product_exact(w, bf16_hi(g.y)) << 16);
        o.z = bf16_of_product_exact(w, bf16_lo(g.z)) | (bf16_of_product_exact(w, bf16_hi(g.z)) << 16);
        o.w = bf16_of_product_exact(w, bf16_lo(g.w)) | (bf16_of_product_exact(w, bf16_hi(g.w)) << 16);
    }
    return o;
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc)
{
    acc = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc);
    acc = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc);
    acc = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc);
    acc = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc);
    acc = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc);
    acc = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc);
    acc = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc);
    acc = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc);
    return acc;
}

// y rows are read once: non-temporal buffer loads (gfx950 "nt" policy bit);
// past the row end they read 0.
__device__ __forceinline__ uint4 load_row_nt(const uint4* row, int nvec, int v)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(row), (short)0, nvec * 16, 0x00020000);
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, 2));
}

__device__ __forceinline__ void keep(uint4& v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

constexpr int kGroup = 8;   // slots whose partial dots are carried together

// A pass covers NT*VPT vectors of the row; lanes past the row end hold
// zeros and store nothing.  STORE: also write grad_y (the fused pass).
template <int NT, int VPT, bool STORE>
__global__ __launch_bounds__(NT)
void combine_backward_kernel(const uint4* __restrict__ g, const uint4* __restrict__ y,
                             const int32_t* __restrict__ slot, const float* __restrict__ w,
                             int nvec, int k, uint4* __restrict__ grad_y,
                             float* __restrict__ grad_w)
{
    __shared__ float red[NT / 64][kGroup];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t sl = lane < k ? slot[t * k + lane] : -1;
    const float wl = lane < k ? (w ? w[t * k + lane] : 1.0f) : 0.0f;
    const uint4* gr = g + t * nvec;
    const bool want_dot = grad_w != nullptr;
    constexpr int kPass = NT * VPT;

    for (int jg = 0; jg < k; jg += kGroup) {
        const int jn = min(kGroup, k - jg);
        float acc[kGroup];
#pragma unroll
        for (int q = 0; q < kGroup; ++q) acc[q] = 0.0f;

        for (int p0 = 0; p0 < nvec; p0 += kPass) {
            uint4 gv[VPT];
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int v = p0 + tid + u * NT;
                gv[u] = v < nvec ? gr[v] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < VPT; ++u) keep(gv[u]);
            GradStat gs[VPT];
#pragma unroll
            for (int u = 0; u < VPT; ++u) gs[u] = STORE ? grad_stat(gv[u]) : GradStat{0.0f, false};
#pragma unroll
            for (int q = 0; q < kGroup; ++q) {
                if (q >= jn) break;
                const int32_t r = __builtin_amdgcn_readlane(sl, jg + q);
                if (r < 0) continue;
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), jg + q));
                const uint4* yr = y + (int64_t)r * nvec;
                const __amdgpu_buffer_rsrc_t dst = buffer_rsrc(grad_y + (int64_t)r * nvec, nvec * 16);
                if (want_dot) {
                    uint4 yv[VPT];
#pragma unroll
                    for (int u = 0; u < VPT; ++u) yv[u] = load_row_nt(yr, nvec, p0 + tid + u * NT);
#pragma unroll
                    for (int u = 0; u < VPT; ++u) acc[q] = dot8(gv[u], yv[u], acc[q]);
                }
                if (STORE) {
#pragma unroll
                    for (int u = 0; u < VPT; ++u) {
                        const int v = p0 + tid + u * NT;
                        if (v < nvec) store_row16(dst, v * 16, scale_row8(wj, gv[u], gs[u]));
                    }
                }
            }
        }

        if (want_dot) {
            // reduce each slot's partial dot over the workgroup
#pragma unroll
            for (int q = 0; q < kGroup; ++q) {
                float v = acc[q];
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
                if (lane == 0) red[wave][q] = v;
            }
            __syncthreads();
            if (tid < jn) {
                float s = 0.0f;
#pragma unroll
                for (int wv = 0; wv < NT / 64; ++wv) s += red[wv][tid];
                const int j = jg + tid;
                const int32_t rj = slot[t * k + j];
                grad_w[t * k + j] = rj >= 0 ? s : 0.0f;
            }
            __syncthreads();
        }
    }
}

// grad_y alone, tiled like the bf16 dispatch: workgroup b maps (XCD-aware)
// to tile `tile` = (token t, tile p of its row) and slot group gi (slots
// 4gi .. 4gi+3); one 16-byte vector per lane, past the row end nothing.
constexpr int kGradYSlots = 4;

__global__ __launch_bounds__(kTileLanes)
void combine_backward_grad_y_tile_kernel(const uint4* __restrict__ g, int nvec, int k, int tpr,
                                         int64_t num_tiles, int groups,
                                         const int32_t* __restrict__ slot,
                                         const float* __restrict__ w, uint4* __restrict__ grad_y)
{
    int64_t tile;
    int gi;
    if (!xcd_tile(blockIdx.x, groups, num_tiles, tile, gi)) return;
    const int64_t t = tile / tpr;
    const int p = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j0 = gi * kGradYSlots;
    // lanes 0..3 of each wavefront hold the group's slots and weights; read
    // back with readlane before any lane diverges
    const bool mine = lane < kGradYSlots && j0 + lane < k;
    const int32_t sl = mine ? slot[t * k + j0 + lane] : -1;
    const float wl = mine ? (w ? w[t * k + j0 + lane] : 1.0f) : 0.0f;
    int32_t r[kGradYSlots];
    float wq[kGradYSlots];
#pragma unroll
    for (int q = 0; q < kGradYSlots; ++q) {
        r[q] = __builtin_amdgcn_readlane(sl, q);
        wq[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), q));
    }
    const int v = p * kTileLanes + tid;
    uint4 d = load_row16<0>(buffer_rsrc(g + t * nvec, nvec * 16), v * 16);
    keep(d);
    const GradStat gs = grad_stat(d);
#pragma unroll
    for (int q = 0; q < kGradYSlots; ++q)
        if (r[q] >= 0 && v < nvec)
            store_row16(buffer_rsrc(grad_y + (int64_t)r[q] * nvec, nvec * 16), v * 16,
                        scale_row8(wq[q], d, gs));
}

}  // namespace

hipError_t launch_combine_backward(const void* grad_out, const void* y, const int32_t* slot,
                                   const float* topk_weights, int64_t num_tokens, int hidden,
                                   int num_topk, void* grad_y, float* grad_topk_weights,
                                   hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const dim3 grid((unsigned)num_tokens);
    const uint4* gg = static_cast<const uint4*>(grad_out);
    const uint4* yy = static_cast<const uint4*>(y);
    uint4* gy = static_cast<uint4*>(grad_y);
    // rows the bf16 dispatch tiles: grad_y in tiles, then grad_w alone
    const int tpr = tiles_per_row(nvec);
    const int groups = (num_topk + kGradYSlots - 1) / kGradYSlots;
    const int64_t num_tiles = num_tokens * tpr;
    const int64_t blocks = (num_tiles + 7) / 8 * 8 * groups;
    const bool split = tile_dispatch(nvec, num_tokens * num_topk) && blocks <= INT32_MAX;
    if (split) {
        hipLaunchKernelGGL(combine_backward_grad_y_tile_kernel, dim3((unsigned)blocks),
                           dim3(kTileLanes), 0, stream, gg, nvec, num_topk, tpr, num_tiles, groups,
                           slot, topk_weights, gy);
        if (grad_topk_weights == nullptr) return hipGetLastError();
    }
    // 64 lanes for short rows; else 128 lanes with the largest VPT <= 8
    // whose pass divides the row (896 = 128*7 at hidden 7168)
    if (nvec <= 64) {
        hipLaunchKernelGGL((combine_backward_kernel<64, 1, true>), grid, dim3(64), 0, stream, gg,
                           yy, slot, topk_weights, nvec, num_topk, gy, grad_topk_weights);
        return hipGetLastError();
    }
    const int fit = nvec / 128;
    int vpt = fit < 1 ? 1 : (fit > 8 ? 8 : fit);
    for (int v = 8; v >= 1; --v) {
        if (nvec % (128 * v) == 0) {
            vpt = v;
            break;
        }
    }
#define EP_CB(V)                                                                             \
    if (split)                                                                               \
        hipLaunchKernelGGL((combine_backward_kernel<128, V, false>), grid, dim3(128), 0, stream, \
                           gg, yy, slot, topk_weights, nvec, num_topk, gy, grad_topk_weights); \
    else                                                                                     \
        hipLaunchKernelGGL((combine_backward_kernel<128, V, true>), grid, dim3(128), 0, stream, \
                           gg, yy, slot, topk_weights, nvec, num_topk, gy, grad_topk_weights)
    switch (vpt) {
    case 1: EP_CB(1); break;
    case 2: EP_CB(2); break;
    case 3: EP_CB(3); break;
    case 4: EP_CB(4); break;
    case 5: EP_CB(5); break;
    case 6: EP_CB(6); break;
    case 7: EP_CB(7); break;
    default: EP_CB(8); break;
    }
#undef EP_CB
    return hipGetLastError();
}

}  // namespace ep

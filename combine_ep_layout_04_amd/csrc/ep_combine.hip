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
// Design (HBM-bound): one workgroup per token; each lane owns 16-byte
// column vectors of the row.  For a vector the k source rows are loaded
// back to back (k independent 16-byte loads in flight per lane before the
// first is consumed), then reduced in j order.  Each loaded byte is used
// once by the lane that loaded it, so the gather goes straight to
// registers; an LDS round trip would add traffic without reuse.  k is a
// template parameter for k <= 8 so the loads are fully unrolled.

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

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int v)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, 0));
}

// K > 0: exactly K = k slots, unrolled.  K == 0: any k (runtime loop).
// Lane j of every wavefront holds slot[t, j] and w[t, j] (k <= 64); they are
// read back as wavefront-uniform values with readlane.
template <int NT, int K>
__global__ __launch_bounds__(NT)
void combine_kernel(const uint4* __restrict__ y, const int32_t* __restrict__ slot,
                    const float* __restrict__ w, int nvec, int k, uint4* __restrict__ out)
{
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kk = K > 0 ? K : k;
    const int32_t sl = lane < kk ? slot[t * kk + lane] : -1;
    const float wl = lane < kk ? (w ? w[t * kk + lane] : 1.0f) : 0.0f;
    uint4* o = out + t * nvec;

    if constexpr (K > 0) {
        // A masked slot reads zeros through an empty resource and gets
        // weight 0, so its term fma(0, 0, acc) leaves acc's value unchanged
        // (at most an accumulated -0 turns into +0) and no branch is needed.
        __amdgpu_buffer_rsrc_t rs[K];
        float g[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(sl, j);
            rs[j] = row_rsrc(y, r, nvec);
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
            g[j] = r >= 0 ? wj : 0.0f;
        }
        for (int v = tid; v < nvec; v += NT) {
            uint4 d[K];
#pragma unroll
            for (int j = 0; j < K; ++j) d[j] = load16(rs[j], v);
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < K; ++j) fma8(acc, g[j], d[j]);
            o[v] = pack8(acc);
        }
    } else {
        for (int v = tid; v < nvec; v += NT) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < kk; ++j) {
                const int32_t r = __builtin_amdgcn_readlane(sl, j);
                if (r < 0) continue;
                const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
                fma8(acc, g, y[(int64_t)r * nvec + v]);
            }
            o[v] = pack8(acc);
        }
    }
}

template <int NT>
void launch_nt(dim3 grid, hipStream_t stream, const uint4* y, const int32_t* slot,
               const float* w, int nvec, int k, uint4* out)
{
    switch (k) {
    case 1: hipLaunchKernelGGL((combine_kernel<NT, 1>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 2: hipLaunchKernelGGL((combine_kernel<NT, 2>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 3: hipLaunchKernelGGL((combine_kernel<NT, 3>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 4: hipLaunchKernelGGL((combine_kernel<NT, 4>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 5: hipLaunchKernelGGL((combine_kernel<NT, 5>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 6: hipLaunchKernelGGL((combine_kernel<NT, 6>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 7: hipLaunchKernelGGL((combine_kernel<NT, 7>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    case 8: hipLaunchKernelGGL((combine_kernel<NT, 8>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    default: hipLaunchKernelGGL((combine_kernel<NT, 0>), grid, dim3(NT), 0, stream, y, slot, w, nvec, k, out); break;
    }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* slot, const float* topk_weights,
                          int64_t num_tokens, int hidden, int num_topk, void* out,
                          hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const dim3 grid((unsigned)num_tokens);
    const uint4* yy = static_cast<const uint4*>(y);
    uint4* oo = static_cast<uint4*>(out);
    if (nvec <= 64)
        launch_nt<64>(grid, stream, yy, slot, topk_weights, nvec, num_topk, oo);
    else
        launch_nt<128>(grid, stream, yy, slot, topk_weights, nvec, num_topk, oo);
    return hipGetLastError();
}

}  // namespace ep

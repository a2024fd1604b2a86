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
//   - one workgroup per token: x[t] is read from HBM exactly once into
//     registers (16-byte loads, `VPT` per lane) and written to each of the
//     token's k destination rows with 16-byte stores, so every wavefront
//     store instruction covers 1 KiB of one contiguous row;
//   - the k slots of a token are wavefront-uniform (scalar loads), so the
//     loop over destinations is a scalar loop with no divergence;
//   - fp8: 16 consecutive lanes hold one 128-channel block (8 bf16 each);
//     amax is reduced across those 16 lanes with cross-lane shuffles, the
//     scale and every quotient are correctly rounded fp32 divisions, and
//     the E4M3 code comes from an integer round-to-nearest-even on the fp32
//     bit pattern (written from the OCP E4M3 definition: bias 7, largest
//     finite 448, codes below 2^-6 are multiples of 2^-9).

#include "ep_internal.h"

namespace ep {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// OCP E4M3 code of f, round-to-nearest-even, magnitudes >= 448 saturate to
// 448, NaN -> S.1111.111, the sign bit is always kept.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;                                   // NaN
    } else if (a >= 0x43E00000u) {
        code = 0x7Eu;                                   // >= 448: saturate
    } else if (a >= 0x3C800000u) {
        // normal E4M3 (>= 2^-6): keep 3 of the 23 mantissa bits with RNE;
        // a carry out of the mantissa bumps the exponent, which is right.
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);                         // rebias 127 -> 7
    } else {
        // below 2^-6 the E4M3 grid is k * 2^-9, k = 0..8 (8 = 2^-6)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

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
            uint4* dst = recv + (int64_t)r * nvec + vb;
#pragma unroll
            for (int u = 0; u < VPT; ++u) dst[u * NT] = buf[u];
        }
    }
    // ragged tail: one vector per lane
    for (int v = full * kPass + tid; v < nvec; v += NT) {
        uint4 d = xr[v];
        keep(d);
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r >= 0) recv[(int64_t)r * nvec + v] = d;
        }
    }
}

// Quantise one 16-byte bf16 vector (8 channels) of a 128-channel block held
// by 16 aligned lanes; all 16 lanes must execute this together.
__device__ __forceinline__ uint2 quantise8(const uint4& d, float& scale)
{
    const float f[8] = {bf16_lo(d.x), bf16_hi(d.x), bf16_lo(d.y), bf16_hi(d.y),
                        bf16_lo(d.z), bf16_hi(d.z), bf16_lo(d.w), bf16_hi(d.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    const float sc = amax / 448.0f;
    scale = sc;
    uint32_t c[8];
    if (amax == 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = 0u;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = e4m3_rne_sat(f[i] / sc);
    }
    uint2 q;
    q.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    q.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    return q;
}

// Each lane quantises 8 channels (one 16-byte bf16 vector); the 16 lanes of
// an aligned lane group share one 128-channel block (nvec is a multiple of
// 16 and so is every pass, so a group is either all in range or all out).
template <int NT, int VPT>
__global__ __launch_bounds__(NT)
void dispatch_fp8_kernel(const uint4* __restrict__ x, int nvec, int k,
                         const int32_t* __restrict__ slot, const float* __restrict__ w,
                         uint2* __restrict__ recv_q, float* __restrict__ recv_s,
                         float* __restrict__ recv_w)
{
    static_assert(NT % 16 == 0, "a 128-channel block is 16 lanes");
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* s = slot + t * k;
    const int32_t sl = token_slots(s, k);
    const int nb = nvec >> 4;

    if (recv_w != nullptr && tid < k && sl >= 0) recv_w[sl] = w[t * k + tid];

    const uint4* xr = x + t * nvec;
    constexpr int kPass = NT * VPT;
    const int full = nvec / kPass;

    for (int p = 0; p < full; ++p) {
        const int vb = p * kPass + tid;
        uint4 d[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) d[u] = xr[vb + u * NT];
        uint2 q[VPT];
        float sc[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) q[u] = quantise8(d[u], sc[u]);
        const bool lead = (tid & 15) == 0;
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r < 0) continue;
            uint2* dq = recv_q + (int64_t)r * nvec + vb;
            float* ds = recv_s + (int64_t)r * nb + (vb >> 4);
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                dq[u * NT] = q[u];
                if (lead) ds[u * (NT / 16)] = sc[u];
            }
        }
    }
    // ragged tail: every lane runs the same trip count so the 16-lane
    // reductions stay converged; out-of-range groups quantise zeros and
    // store nothing
    for (int vb = full * kPass; vb < nvec; vb += NT) {
        const int v = vb + tid;
        const bool live = v < nvec;
        uint4 d = make_uint4(0u, 0u, 0u, 0u);
        if (live) d = xr[v];
        float sc;
        const uint2 q = quantise8(d, sc);
        if (!live) continue;
        for (int j = 0; j < k; ++j) {
            const int32_t r = lane_value(sl, j);
            if (r < 0) continue;
            recv_q[(int64_t)r * nvec + v] = q;
            if ((v & 15) == 0) recv_s[(int64_t)r * nb + (v >> 4)] = sc;
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
    const Shape sh = pick_shape(nvec);
    const dim3 grid((unsigned)num_tokens);
    EP_DISPATCH_CASES(dispatch_bf16_kernel, static_cast<const uint4*>(x), nvec, num_topk, slot,
                      topk_weights, static_cast<uint4*>(recv_x), recv_weights)
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const void* x, int64_t num_tokens, int hidden, int num_topk,
                               const int32_t* slot, const float* topk_weights, void* recv_q,
                               float* recv_scales, float* recv_weights, hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const Shape sh = pick_shape(nvec);
    const dim3 grid((unsigned)num_tokens);
    EP_DISPATCH_CASES(dispatch_fp8_kernel, static_cast<const uint4*>(x), nvec, num_topk, slot,
                      topk_weights, static_cast<uint2*>(recv_q), recv_scales, recv_weights)
    return hipGetLastError();
}

}  // namespace ep

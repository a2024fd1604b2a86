// ep_cast.h -- the 8-bit cast of bf16 channels in blocks of 128 (OCP E4M3
// or E5M2 codes, with an fp32, power-of-two or UE8M0 block scale), shared
// by the expanded dispatch and the once-per-rank dispatch.
//
// Passages: NCCL EP page, ncclEpDispatch (fp8 output with hidden/128 fp32
// scales per token, scale block 128; the low-latency branch casts inside
// the dispatch, with round_scale and use_ue8m0); DeepEP page, ElasticBuffer
// (use_fp8_dispatch).
//
// Each lane casts one "unit" of 16 channels (two 16-byte loads in, one
// 16-byte store out), so 8 aligned lanes hold a block and its amax is an
// 8-lane reduction by DPP lane moves.  With fp32 scales the quotients use
// Markstein's correction (P. Markstein, IBM J. Res. Dev. 34(1), 1990) from
// one reciprocal per block; the encoders are integer round-to-nearest-even
// on the fp32 bit pattern, written from the OCP 8-bit format definitions.

#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ep {

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



// E4M3 code of a finite q with 0 <= q < 464 (no saturation or NaN case can
// arise when |x| <= amax): normal range by integer RNE on the bit pattern,
// below 2^-6 by one float add that rounds to a multiple of 2^-9 (adding
// 2^14 leaves exactly 2^-9 per unit in the last place).
__device__ __forceinline__ uint32_t e4m3_small_nonneg(float q)
{
    const uint32_t a = __float_as_uint(q);
    const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    const uint32_t tiny = __float_as_uint(q + 16384.0f) - 0x46800000u;
    return a >= 0x3C800000u ? normal : tiny;
}

// OCP E5M2 (bias 15, 2 mantissa bits, largest finite 57344 = 1.75 * 2^15,
// codes below 2^-14 are multiples of 2^-16), written from its definition.
// Finite q with 0 <= q < 61440: keep 2 of 23 mantissa bits with RNE; below
// 2^-14 add 2^7, whose unit in the last place is 2^-16.
__device__ __forceinline__ uint32_t e5m2_small_nonneg(float q)
{
    const uint32_t a = __float_as_uint(q);
    const uint32_t normal = ((a + 0xFFFFFu + ((a >> 21) & 1u)) >> 21) - (112u << 2);
    const uint32_t tiny = __float_as_uint(q + 128.0f) - 0x43000000u;
    return a >= 0x38800000u ? normal : tiny;
}

// Any q: saturation to 57344 (infinities included), NaN -> S.11111.11.
__device__ __forceinline__ uint32_t e5m2_rne_sat(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u)
        code = 0x7Fu;
    else if (a >= 0x47600000u)
        code = 0x7Bu;
    else if (a >= 0x38800000u)
        code = ((a + 0xFFFFFu + ((a >> 21) & 1u)) >> 21) - (112u << 2);
    else
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
    return sign | code;
}

// Output formats and scale modes of the 8-bit cast.
constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;
constexpr int kScaleFp32 = 0;   // scale = amax / max_finite
constexpr int kScalePow2 = 1;   // smallest power of two >= amax / max_finite, fp32
constexpr int kScaleUe8m0 = 2;  // the same power of two as one exponent byte

template <int FMT>
__device__ __forceinline__ float max_finite() { return FMT == kE5M2 ? 57344.0f : 448.0f; }

template <int FMT>
__device__ __forceinline__ uint32_t encode_nonneg(float q)
{
    return FMT == kE5M2 ? e5m2_small_nonneg(q) : e4m3_small_nonneg(q);
}

template <int FMT>
__device__ __forceinline__ uint32_t encode_any(float q)
{
    return FMT == kE5M2 ? e5m2_rne_sat(q) : e4m3_rne_sat(q);
}

constexpr int kLanesPerBlock = 8;   // 16 channels per lane, 128 per block

// DPP lane moves within a row of 16 lanes (gfx9 DPP control codes):
// quad_perm [1,0,3,2] swaps neighbours, quad_perm [2,3,0,1] swaps pairs of a
// quad, row_half_mirror reverses each group of 8 lanes.  Moved through the
// data-parallel ALU instead of LDS (ds_bpermute).
constexpr int kDppSwap1 = 0xB1;
constexpr int kDppSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum of v over each aligned group of 8 lanes, returned to all 8.  Max
// is order-free, so swap-1, swap-2 and a mirror of the 8 lanes (which pairs
// each quad with the other) reach every lane of the group.  All 8 lanes of
// a group must be active together (they always take the same branch here).
__device__ __forceinline__ uint32_t group8_max_u32(uint32_t v)
{
    v = max(v, dpp_move<kDppSwap1>(v));
    v = max(v, dpp_move<kDppSwap2>(v));
    return max(v, dpp_move<kDppHalfMirror>(v));
}

__device__ __forceinline__ float group8_max_f32(float v)
{
    v = fmaxf(v, __uint_as_float(dpp_move<kDppSwap1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_move<kDppSwap2>(__float_as_uint(v))));
    return fmaxf(v, __uint_as_float(dpp_move<kDppHalfMirror>(__float_as_uint(v))));
}

// Smallest e with 2^e >= s (s > 0 finite): frexp gives s = m * 2^ex with
// m in [0.5, 1); s is a power of two exactly when m == 0.5.
__device__ __forceinline__ int ceil_log2(float s)
{
    int ex;
    const float m = frexpf(s, &ex);
    return m == 0.5f ? ex - 1 : ex;
}

// Exponent of a power-of-two scale: the smallest e with 2^e >= amax / fmax,
// the exact quotient, for finite amax > 0.  amax is a bf16 value (8
// significant bits) and fmax is 7 * 2^n, so the quotient is a power of two
// only when the division is exact, and otherwise lies at least 2^-8
// (relative) away from one: a correctly rounded fp32 quotient decides e, as
// long as it is normal.  For amax below 2^-64 the fp32 quotient would be
// subnormal (amax 2^-133 over 57344 rounds down onto 2^-149, one binade
// short, and the codes would then overflow), so such an amax is scaled by
// 2^64 first; amax >= 2^-133 keeps the scaled quotient normal.
__device__ __forceinline__ int pow2_exponent(float amax, float fmax)
{
    const bool tiny = amax < 0x1p-64f;
    const int e = ceil_log2((tiny ? amax * 0x1p64f : amax) / fmax);
    return tiny ? e - 64 : e;
}

// Codes (16 bytes) and block scale for the 16 channels in d0:d1; the 8
// aligned lanes of one 128-channel block must execute this together.  The
// scale comes back as fp32 (modes 0, 1) or as the UE8M0 byte in its low
// bits (mode 2).
template <int FMT, int SM>
__device__ __forceinline__ uint4 quantise16(const uint4& d0, const uint4& d1, uint32_t& scale_bits)
{
    const float f[16] = {bf16_lo(d0.x), bf16_hi(d0.x), bf16_lo(d0.y), bf16_hi(d0.y),
                         bf16_lo(d0.z), bf16_hi(d0.z), bf16_lo(d0.w), bf16_hi(d0.w),
                         bf16_lo(d1.x), bf16_hi(d1.x), bf16_lo(d1.y), bf16_hi(d1.y),
                         bf16_lo(d1.z), bf16_hi(d1.z), bf16_lo(d1.w), bf16_hi(d1.w)};
    // max |x| as an unsigned compare of the magnitude bits (same order as
    // the values; a NaN compares above infinity)
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(f[i]) & 0x7FFFFFFFu);
    m = group8_max_u32(m);

    const float fmax = max_finite<FMT>();
    uint32_t c[16];
    if (SM == kScaleFp32 && m >= 0x17800000u && m < 0x7F800000u) {
        // 2^-80 <= amax < inf: Markstein-corrected quotients
        const float amax = __uint_as_float(m);
        const float sc = amax / fmax;
        const float y = 1.0f / sc;
        scale_bits = __float_as_uint(sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ax = fabsf(f[i]);
            const float q0 = ax * y;
            const float r = __builtin_fmaf(-q0, sc, ax);
            const float q = __builtin_fmaf(r, y, q0);
            c[i] = encode_nonneg<FMT>(q) | ((__float_as_uint(f[i]) >> 24) & 0x80u);
        }
    } else if (SM != kScaleFp32 && m > 0u && m < 0x7F800000u) {
        // finite nonzero amax, power-of-two scale: q = x * 2^-e is exact and
        // |q| <= max_finite
        int e = pow2_exponent(__uint_as_float(m), fmax);
        if (SM == kScaleUe8m0 && e < -127) e = -127;
        scale_bits = SM == kScaleUe8m0 ? (uint32_t)(e + 127) : __float_as_uint(ldexpf(1.0f, e));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            c[i] = encode_nonneg<FMT>(ldexpf(fabsf(f[i]), -e)) |
                   ((__float_as_uint(f[i]) >> 24) & 0x80u);
    } else {
        // zero, tiny (fp32 mode), infinite or NaN-holding blocks: amax
        // ignores NaN (an IEEE max), plain division (or exact power-of-two
        // scaling for a finite amax)
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = group8_max_f32(amax);
        const bool pow2 = SM != kScaleFp32 && amax > 0.0f && amax < __builtin_inff();
        int e = 0;
        float sc = amax / fmax;
        if (pow2) {
            e = pow2_exponent(amax, fmax);
            if (SM == kScaleUe8m0 && e < -127) e = -127;
            sc = ldexpf(1.0f, e);
        }
        if (SM == kScaleUe8m0)
            scale_bits = amax == 0.0f ? 0u : (pow2 ? (uint32_t)(e + 127) : 0xFFu);
        else
            scale_bits = __float_as_uint(sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float q = pow2 ? ldexpf(f[i], -e) : f[i] / sc;
            // a NaN quotient (NaN x, or infinite x over an infinite scale)
            // is S.1111111 with the sign of x, whatever NaN the divide made
            const uint32_t sx = (__float_as_uint(f[i]) >> 24) & 0x80u;
            c[i] = amax == 0.0f ? 0u : (q != q ? (0x7Fu | sx) : encode_any<FMT>(q));
        }
    }
    uint4 q;
    q.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    q.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    q.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
    q.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
    return q;
}

}  // namespace ep

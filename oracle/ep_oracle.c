/*
 * ep_oracle.c -- plain, slow CPU oracle for MoE token layout, dispatch and
 * combine on one device's share.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Built with gcc, -O2 -ffp-contract=off, no fast-math, so every float
 * operation below is one IEEE-754 operation in the stated precision.
 *
 * What is computed, and the passages it follows:
 *
 *  - Layout (NCCL EP page, nccl_ep.cc, ncclEpCreateHandle "Step 3:
 *    metadata_preprocessing"; DeepEP page, "Prefix Sum Interpretation for
 *    Expert Token Counts" and dispatch() option do_expand, "one slot per
 *    token per expert"; NeMo fused_a2a page, HybridEPDispatch topk_idx with
 *    -1 for unused slots).  A stable counting sort of the flat pair index
 *    i = t*k + j by expert id: counts, exclusive offsets, the destination
 *    row of every pair and the source token of every destination row.
 *
 *  - Dispatch, bf16 (NCCL EP page, ncclEpDispatch; DeepEP page, dispatch()
 *    returns recv_x and recv_topk_weights): a byte copy of token row t to
 *    every destination row of its unmasked pairs.
 *
 *  - Dispatch, fp8 (NCCL EP page: per-token scale bytes hidden/128 * 4,
 *    scales tensor [.., .., hidden/128] fp32 with scale_block_size 128,
 *    datatype ncclFloat8e4m3): per 128-channel block, amax in fp32,
 *    scale = fl32(amax / 448), q = e4m3fn(fl32(x / scale)) with
 *    round-to-nearest-even and saturation to +-448.  The encoder is written
 *    from the OCP 8-bit floating point definition of E4M3 (bias 7, no
 *    infinities, S.1111.111 is NaN, largest finite 448).
 *
 *  - Combine (NCCL EP page, ncclEpCombine low-latency branch: weighted by
 *    topk_weights [T,k]; DeepEP page, combine()): out[t] = sum over unmasked
 *    j of w[t,j] * y[slot[t,j]], summed in fp64 in ascending j and rounded
 *    once to bf16 (round-to-nearest-even).  A NULL weight array means unit
 *    weights (the unweighted forward combine of the high-throughput path).
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t bits_of_float_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/*
 * Round a double to the nearest bf16 value, ties to an even significand.
 * bf16 has 8 significant bits and the float32 exponent range: normals down
 * to 2^-126, subnormals in steps of 2^-133, largest finite (2 - 2^-7)*2^127.
 * The quantum at |d| is 2^(e-7) where 2^e <= |d| < 2^(e+1), or 2^-133 below
 * 2^-126; |d| / quantum is rounded to an integer with nearbyint (the default
 * rounding mode is to-nearest-even), which makes the rounding exact.
 */
uint16_t oracle_bf16_from_double(double d)
{
    if (isnan(d))
        return (uint16_t)(signbit(d) ? 0xFFC0u : 0x7FC0u);
    int neg = signbit(d) != 0;
    double a = fabs(d);
    if (a == 0.0)
        return (uint16_t)(neg ? 0x8000u : 0x0000u);
    int ex;
    (void)frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;               /* 2^e <= a < 2^(e+1) */
    int qexp = (e < -126) ? -133 : e - 7;
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    if (r >= ldexp(1.0, 128))     /* beyond the largest finite: overflow */
        return (uint16_t)(neg ? 0xFF80u : 0x7F80u);
    float rf = (float)r;          /* exact: r has <= 8 significant bits */
    uint16_t h = bits_of_float_hi(rf);
    return (uint16_t)(neg ? (h | 0x8000u) : h);
}

/* --------------------------------------------------------------- e4m3 -- */

/* OCP E4M3 value of code c: (-1)^s 2^(e-7) (1 + m/8) for e > 0,
 * (-1)^s 2^-6 (m/8) for e == 0, NaN for S.1111.111. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/*
 * Nearest E4M3 code to v, ties to the even code, magnitudes above 448
 * saturated to 448 (the "satfinite" conversion).  The sign is kept, so -0
 * and negative values that round to zero give 0x80.  NaN gives S.1111.111.
 * Below 2^-6 the step is 2^-9 and the code is simply round(|v| * 2^9)
 * (a result of 8 is the code of 2^-6, the smallest normal).  From 2^-6 up
 * the code is (e+7)*8 + round((|v|/2^e - 1) * 8), where a mantissa that
 * rounds up to 8 carries into the exponent field.
 */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a > 448.0)
        a = 448.0;
    int code;
    if (a < ldexp(1.0, -6)) {
        code = (int)nearbyint(ldexp(a, 9));
    } else {
        int ex;
        (void)frexp(a, &ex);
        int e = ex - 1;                             /* -6 <= e <= 8 */
        double mant = ldexp(a, -e) - 1.0;           /* in [0, 1), exact */
        int m = (int)nearbyint(mant * 8.0);         /* exact scaling */
        code = (e + 7) * 8 + m;
    }
    return (uint8_t)(sign | (uint8_t)code);
}

/* ------------------------------------------------------------- layout -- */

/*
 * Stable counting sort of the pairs i = t*k + j by expert e = topk_idx[i].
 * e == -1 is a masked slot; any e outside [-1, E) is counted in
 * *num_invalid and also treated as masked.  Outputs:
 *   counts[e]      number of unmasked pairs routed to e
 *   offsets[e]     exclusive prefix sum of counts, offsets[E] = N
 *   slot[i]        destination row of pair i in [0, N), or -1 if masked;
 *                  pairs of one expert keep their flat order
 *   src[r]         source token of destination row r < N (may be NULL)
 */
void oracle_layout(const int64_t *topk_idx, int64_t T, int k, int E,
                   int32_t *counts, int32_t *offsets, int32_t *slot,
                   int32_t *src, int32_t *num_invalid)
{
    int64_t P = T * (int64_t)k;
    int32_t bad = 0;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < P; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E)
            counts[e] += 1;
        else if (e != -1)
            bad += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    /* second pass: hand out rows in increasing flat order per expert */
    int32_t *cursor = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t i = 0; i < P; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E) {
            int32_t r = cursor[e]++;
            slot[i] = r;
            if (src)
                src[r] = (int32_t)(i / k);
        } else {
            slot[i] = -1;
        }
    }
    free(cursor);
    if (num_invalid)
        *num_invalid = bad;
}

/* ----------------------------------------------------------- dispatch -- */

/* recv_x[slot[t,j], :] = x[t, :] for every unmasked pair (bf16 bytes), and
 * recv_w[slot[t,j]] = topk_weights[t,j] when both are given. */
void oracle_dispatch_bf16(const uint16_t *x, int64_t T, int H, int k,
                          const int32_t *slot, const float *topk_weights,
                          uint16_t *recv_x, float *recv_w)
{
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[t * k + j];
            if (r < 0)
                continue;
            memcpy(recv_x + (int64_t)r * H, x + t * H, (size_t)H * sizeof(uint16_t));
            if (recv_w && topk_weights)
                recv_w[r] = topk_weights[t * k + j];
        }
}

/* Per token t and channel block b of 128: amax = max |x| (NaN ignored),
 * scale = fl32(amax/448), q = e4m3(fl32(x/scale)); amax == 0 gives scale 0
 * and all-zero codes; a NaN quotient gives 0x7F with the sign of x.  The same codes and scales go to every unmasked row of t:
 * recv_q [N, H] bytes, recv_scales [N, H/128] fp32. */
void oracle_dispatch_fp8(const uint16_t *x, int64_t T, int H, int k,
                         const int32_t *slot, const float *topk_weights,
                         uint8_t *recv_q, float *recv_scales, float *recv_w)
{
    int nb = H / 128;
    uint8_t *row_q = (uint8_t *)malloc((size_t)H);
    float *row_s = (float *)malloc((size_t)nb * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *xr = x + t * H;
        for (int b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) {
                float v = (float)oracle_bf16_to_double(xr[b * 128 + c]);
                float av = fabsf(v);
                if (av > amax)
                    amax = av;
            }
            float scale = amax / 448.0f;
            row_s[b] = scale;
            for (int c = 0; c < 128; ++c) {
                if (amax == 0.0f) {
                    row_q[b * 128 + c] = 0x00;
                } else {
                    float v = (float)oracle_bf16_to_double(xr[b * 128 + c]);
                    float q = v / scale;
                    /* a NaN quotient (NaN x, or infinite x over an infinite
                     * scale) is S.1111.111 with the sign of x */
                    row_q[b * 128 + c] = isnan(q) ? (uint8_t)(0x7F | (signbit(v) ? 0x80 : 0))
                                                  : oracle_e4m3_encode(q);
                }
            }
        }
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[t * k + j];
            if (r < 0)
                continue;
            memcpy(recv_q + (int64_t)r * H, row_q, (size_t)H);
            memcpy(recv_scales + (int64_t)r * nb, row_s, (size_t)nb * sizeof(float));
            if (recv_w && topk_weights)
                recv_w[r] = topk_weights[t * k + j];
        }
    }
    free(row_q);
    free(row_s);
}

/* ------------------------------------------------------------ combine -- */

/* out[t, c] = bf16( sum_{j ascending, slot >= 0} w[t,j] * y[slot[t,j], c] ),
 * each product and the running sum in fp64, one rounding to bf16 at the
 * end; w == NULL means w = 1; a token with no unmasked pair gets +0. */
void oracle_combine(const uint16_t *y, const int32_t *slot, const float *topk_weights,
                    int64_t T, int H, int k, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t r = slot[t * k + j];
                if (r < 0)
                    continue;
                double w = topk_weights ? (double)topk_weights[t * k + j] : 1.0;
                acc += w * oracle_bf16_to_double(y[(int64_t)r * H + c]);
            }
            out[t * H + c] = oracle_bf16_from_double(acc);
        }
}

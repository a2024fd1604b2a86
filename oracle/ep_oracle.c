/*
 * ep_oracle.c -- plain, slow CPU oracle for MoE token layout, dispatch and
 * combine on one device's share.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Built with gcc, -O2 -ffp-contract=off, no fast-math, so every float
 * operation below is one IEEE-754 operation in the stated precision.  The
 * same source built with -fopenmp (liboracle_omp.so) runs the bf16 dispatch
 * and combine token loops on all host cores: the benchmark's multi-core CPU
 * baseline, with the same results (tokens write disjoint rows).
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
 *
 *  - The per-(token, rank) path (NCCL EP page, the high-throughput handle's
 *    routing bitmap, sparse_to_dense_map, local_expert_routing_map and
 *    num_tokens_for_experts): the routing bitmap of topk_idx, the receive
 *    rows of every (token, destination rank) pair, the receiving rank's
 *    per-row local expert map, and a dispatch / combine that moves each
 *    token once per rank.  Defined in the last section of this file.
 */

#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
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

/* OCP E5M2 value of code c: (-1)^s 2^(e-15) (1 + m/4) for 0 < e < 31,
 * (-1)^s 2^-14 (m/4) for e == 0; e == 31 is infinity (m == 0) or NaN. */
double oracle_e5m2_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = (e == 0) ? ldexp((double)m / 4.0, -14) : ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -mag : mag;
}

/* Nearest E5M2 code to v, ties to the even code, magnitudes above the
 * largest finite value 57344 (and infinities) saturated to it; sign kept;
 * NaN gives S.11111.11.  Below 2^-14 the step is 2^-16. */
uint8_t oracle_e5m2_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a > 57344.0)
        a = 57344.0;
    int code;
    if (a < ldexp(1.0, -14)) {
        code = (int)nearbyint(ldexp(a, 16));
    } else {
        int ex;
        (void)frexp(a, &ex);
        int e = ex - 1;                             /* -14 <= e <= 15 */
        double mant = ldexp(a, -e) - 1.0;
        int m = (int)nearbyint(mant * 4.0);
        code = (e + 15) * 4 + m;
    }
    return (uint8_t)(sign | (uint8_t)code);
}

/* ------------------------------------------------------------- layout -- */

static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

/*
 * Stable counting sort of the pairs i = t*k + j by expert e = topk_idx[i],
 * with the segment placement options of the pages' expanded layouts:
 *
 *  - packed (expert_capacity == 0): expert e's rows start at
 *      start[e] = sum_{e' < e} align_up(count[e'], alignment),
 *    i.e. every segment starts on a multiple of `alignment` (DeepEP page,
 *    "Prefix Sum Interpretation for Expert Token Counts": in expand mode
 *    start = align(psum[i-1], expert_alignment), end = psum[i]; NeMo page,
 *    HybridEP pad_multiple).  alignment == 1 is the compact layout.
 *  - fixed stride (expert_capacity > 0): expert e owns rows
 *    [e * cap, (e + 1) * cap) (NCCL EP page, ncclEpDispatch low-latency
 *    branch: recv_x [num_local_experts, capacity, hidden] with a per-expert
 *    recv_count).  Pairs past an expert's capacity, in flat order, are
 *    dropped: slot -1, counted in *num_dropped.
 *
 * e == -1 is a masked slot; any e outside [-1, E) is counted in
 * *num_invalid and also treated as masked.  Outputs:
 *   counts[e]      rows of expert e that were placed
 *   offsets[e]     first row of expert e; offsets[E] = total rows of the
 *                  layout (padding included)
 *   slot[i]        destination row of pair i, or -1 (masked / dropped);
 *                  pairs of one expert keep their flat order
 *   src[r]         source token of every placed row r (may be NULL); rows
 *                  nothing maps to are not written
 */
void oracle_layout_ex(const int64_t *topk_idx, int64_t T, int k, int E, int alignment,
                      int64_t expert_capacity, int32_t *counts, int32_t *offsets,
                      int32_t *slot, int32_t *src, int32_t *num_invalid, int32_t *num_dropped)
{
    int64_t P = T * (int64_t)k;
    int32_t bad = 0, dropped = 0;
    int64_t *raw = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *start = (int64_t *)malloc((size_t)E * sizeof(int64_t));
    int64_t *cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < P; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E)
            raw[e] += 1;
        else if (e != -1)
            bad += 1;
    }
    int64_t acc = 0;
    for (int e = 0; e < E; ++e) {
        if (expert_capacity > 0) {
            start[e] = (int64_t)e * expert_capacity;
            counts[e] = (int32_t)(raw[e] < expert_capacity ? raw[e] : expert_capacity);
        } else {
            start[e] = acc;
            acc += align_up(raw[e], alignment);
            counts[e] = (int32_t)raw[e];
        }
        offsets[e] = (int32_t)start[e];
    }
    offsets[E] = (int32_t)(expert_capacity > 0 ? (int64_t)E * expert_capacity : acc);
    /* second pass: hand out rows in increasing flat order per expert */
    for (int64_t i = 0; i < P; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E) {
            int64_t local = cursor[e]++;
            if (expert_capacity > 0 && local >= expert_capacity) {
                slot[i] = -1;
                dropped += 1;
                continue;
            }
            int32_t r = (int32_t)(start[e] + local);
            slot[i] = r;
            if (src)
                src[r] = (int32_t)(i / k);
        } else {
            slot[i] = -1;
        }
    }
    free(raw);
    free(start);
    free(cursor);
    if (num_invalid)
        *num_invalid = bad;
    if (num_dropped)
        *num_dropped = dropped;
}

/* The compact layout: alignment 1, no capacity. */
void oracle_layout(const int64_t *topk_idx, int64_t T, int k, int E,
                   int32_t *counts, int32_t *offsets, int32_t *slot,
                   int32_t *src, int32_t *num_invalid)
{
    oracle_layout_ex(topk_idx, T, k, E, 1, 0, counts, offsets, slot, src, num_invalid, NULL);
}

/* ----------------------------------------------------------- dispatch -- */

/* recv_x[slot[t,j], :] = x[t, :] for every unmasked pair (bf16 bytes), and
 * recv_w[slot[t,j]] = topk_weights[t,j] when both are given. */
void oracle_dispatch_bf16(const uint16_t *x, int64_t T, int H, int k,
                          const int32_t *slot, const float *topk_weights,
                          uint16_t *recv_x, float *recv_w)
{
    /* tokens write disjoint rows: the loop may run in parallel (only in the
     * -fopenmp build that serves as the multi-core CPU baseline; the
     * oracle itself is built without it and runs this loop in order) */
#pragma omp parallel for schedule(static)
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
    /* each token's row is its own: parallel only in the -fopenmp build */
#pragma omp parallel for schedule(static)
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

/* Threads the multi-core baseline build runs its parallel loops on (1 in the
 * oracle's own build, which has no OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    int n = 0;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}

/* ----------------------------------------------------------- backward -- */

/*
 * Backward of the weighted combine (DeepEP page, "MoE Dispatch and Combine
 * for Training/Inference with ElasticBuffer": the backward of combine is a
 * dispatch; NeMo page, HybridEPCombine.backward redispatches the combined-
 * output gradients through the saved layout).  With out[t] = sum_j
 * w[t,j] * y[slot[t,j]]:
 *   grad_y[slot[t,j], c] = bf16( w[t,j] * g[t,c] )   (exact product in fp64,
 *                                                     one rounding)
 *   grad_w[t,j] = fl32( sum_c g[t,c] * y[slot[t,j], c] )   (fp64 sum)
 * Masked pairs write no row and get grad_w 0.  w == NULL means unit
 * weights; grad_w may be NULL (then y is not read).  A NaN product (a NaN
 * weight or gradient, or 0 * inf) gives the canonical quiet NaN 0x7FC0, the
 * bf16 NaN torch's float-to-bf16 cast returns for any NaN: the sign of a
 * NaN that a multiply makes is not the same on every machine.
 */
void oracle_combine_backward(const uint16_t *g, const uint16_t *y, const int32_t *slot,
                             const float *topk_weights, int64_t T, int H, int k,
                             uint16_t *grad_y, float *grad_w)
{
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[t * k + j];
            if (r < 0) {
                if (grad_w)
                    grad_w[t * k + j] = 0.0f;
                continue;
            }
            double w = topk_weights ? (double)topk_weights[t * k + j] : 1.0;
            double dot = 0.0;
            for (int c = 0; c < H; ++c) {
                double gv = oracle_bf16_to_double(g[t * H + c]);
                double prod = w * gv;               /* exact: 24 + 8 significant bits */
                grad_y[(int64_t)r * H + c] = isnan(prod) ? 0x7FC0u : oracle_bf16_from_double(prod);
                if (grad_w)
                    dot += gv * oracle_bf16_to_double(y[(int64_t)r * H + c]);
            }
            if (grad_w)
                grad_w[t * k + j] = (float)dot;
        }
}

/*
 * Backward of dispatch (DeepEP page, same section: the backward of dispatch
 * is a combine, which also returns the reduced weight gradients):
 *   grad_x[t] = bf16( sum_j grad_recv[slot[t,j]] )          (unit weights)
 *   grad_w[t,j] = grad_recv_w[slot[t,j]], 0 if masked
 * grad_recv_w / grad_w may be NULL.
 */
void oracle_dispatch_backward(const uint16_t *grad_recv, const float *grad_recv_w,
                              const int32_t *slot, int64_t T, int H, int k, uint16_t *grad_x,
                              float *grad_w)
{
    oracle_combine(grad_recv, slot, NULL, T, H, k, grad_x);
    if (grad_w && grad_recv_w)
        for (int64_t i = 0; i < T * (int64_t)k; ++i)
            grad_w[i] = slot[i] >= 0 ? grad_recv_w[slot[i]] : 0.0f;
}

/* ------------------------------------------------------ fp8 variants -- */

/*
 * Dispatch with an 8-bit float cast, in the variants the pages name (NCCL EP
 * page, ncclEpDispatch: datatypes ncclFloat8e4m3 / ncclFloat8e5m2; the
 * low-latency kernel's round_scale and use_ue8m0 arguments; DeepEP page,
 * dispatch() FP8 data with scale factors):
 *   format 0: OCP E4M3 (largest finite 448), 1: OCP E5M2 (57344)
 *   scale_mode 0: scale = fl32(amax / max_finite), q = code(fl32(x / scale))
 *   scale_mode 1: power-of-two scale 2^e, e the smallest integer with
 *                 2^e >= amax / max_finite (the exact quotient), stored as
 *                 fp32; q = code(x * 2^-e) (exact, and never above
 *                 max_finite)
 *   scale_mode 2: as 1, stored as one UE8M0 byte e + 127 with e clamped to
 *                 -127 (the byte's smallest value)
 * amax ignores NaN.  amax == 0: codes 0, scale 0 (fp32) or byte 0.  An
 * infinite amax: scale inf (fp32) or byte 0xFF, finite x encode to signed
 * zero.  A NaN quotient is S.1111111 (0x7F) with the sign of x.
 * recv_scales is fp32 [rows, H/128] for modes 0-1 and bytes for mode 2.
 */
static uint8_t encode_fmt(int format, float q) { return format ? oracle_e5m2_encode(q) : oracle_e4m3_encode(q); }

void oracle_dispatch_quant(const uint16_t *x, int64_t T, int H, int k, const int32_t *slot,
                           const float *topk_weights, int format, int scale_mode,
                           uint8_t *recv_q, void *recv_scales, float *recv_w)
{
    int nb = H / 128;
    float fmax = format ? 57344.0f : 448.0f;
    uint8_t *row_q = (uint8_t *)malloc((size_t)H);
    float *row_s = (float *)malloc((size_t)nb * sizeof(float));
    uint8_t *row_b = (uint8_t *)malloc((size_t)nb);
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *xr = x + t * H;
        for (int b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) {
                float av = fabsf((float)oracle_bf16_to_double(xr[b * 128 + c]));
                if (av > amax)
                    amax = av;
            }
            int e = 0;
            float scale;
            if (scale_mode == 0 || amax == 0.0f || isinf(amax)) {
                scale = amax / fmax;
            } else {
                /* e from the quotient amax / max_finite in double: amax is a
                 * bf16 value (8 significant bits) and max_finite is 7 * 2^n,
                 * so the quotient is a power of two only when the division is
                 * exact, and otherwise lies at least 2^-11 (relative) away
                 * from one; its double rounding (2^-53) never crosses a power
                 * of two.  The fp32 quotient would not do: below 2^-126 it
                 * keeps too few bits, and for amax 2^-133 over 57344 it
                 * rounds down onto 2^-149, one binade short. */
                int ex;
                double s0 = (double)amax / (double)fmax;
                double f = frexp(s0, &ex);              /* s0 = f * 2^ex, f in [0.5, 1) */
                e = (f == 0.5) ? ex - 1 : ex;           /* smallest e with 2^e >= s0 */
                if (scale_mode == 2 && e < -127)
                    e = -127;
                scale = ldexpf(1.0f, e);
            }
            row_s[b] = scale;
            row_b[b] = amax == 0.0f ? 0 : (isinf(amax) ? 0xFF : (uint8_t)(e + 127));
            for (int c = 0; c < 128; ++c) {
                float v = (float)oracle_bf16_to_double(xr[b * 128 + c]);
                if (amax == 0.0f) {
                    row_q[b * 128 + c] = 0x00;
                    continue;
                }
                float q = (scale_mode == 0 || isinf(amax)) ? v / scale : ldexpf(v, -e);
                row_q[b * 128 + c] = isnan(q) ? (uint8_t)(0x7F | (signbit(v) ? 0x80 : 0))
                                              : encode_fmt(format, q);
            }
        }
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[t * k + j];
            if (r < 0)
                continue;
            memcpy(recv_q + (int64_t)r * H, row_q, (size_t)H);
            if (scale_mode == 2)
                memcpy((uint8_t *)recv_scales + (int64_t)r * nb, row_b, (size_t)nb);
            else
                memcpy((float *)recv_scales + (int64_t)r * nb, row_s, (size_t)nb * sizeof(float));
            if (recv_w && topk_weights)
                recv_w[r] = topk_weights[t * k + j];
        }
    }
    free(row_q);
    free(row_s);
    free(row_b);
}

/*
 * Dispatch of an input that is already 8-bit floats with per-128 fp32
 * scales (NCCL EP page, ncclEpDispatch high-throughput branch: FP8 is
 * detected from the input datatype and the scales tensor comes with it;
 * DeepEP page, dispatch() x as a (data, scale_factors) tuple): the code row
 * and scale row of token t are copied to every unmasked slot.
 */
void oracle_dispatch_prequant(const uint8_t *xq, const float *xs, int64_t T, int H, int k,
                              const int32_t *slot, const float *topk_weights, uint8_t *recv_q,
                              float *recv_s, float *recv_w)
{
    int nb = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[t * k + j];
            if (r < 0)
                continue;
            memcpy(recv_q + (int64_t)r * H, xq + t * H, (size_t)H);
            memcpy(recv_s + (int64_t)r * nb, xs + t * nb, (size_t)nb * sizeof(float));
            if (recv_w && topk_weights)
                recv_w[r] = topk_weights[t * k + j];
        }
}

/* ------------------------------------------ per-(token, rank) layout -- */

/*
 * The non-expanded path (NCCL EP page, nccl_ep.cc: the high-throughput
 * handle's routing structures global_routing_map, sparse_to_dense_map,
 * local_expert_routing_map and num_tokens_for_experts, and the
 * high-throughput branch of ncclEpCreateHandle: Step 1 converts topk_idx to
 * the bitmap, Step 2 all-gathers it, Step 3 runs the metadata preprocessing
 * with the per-expert receive counter).  A token travels to a rank once, no
 * matter how many of that rank's experts it selected.
 *
 * G ranks; rank d owns experts [d*El, (d+1)*El), El = E / G.  Every rank
 * contributes T rows to the all-gathered map, so the global token
 * g = s*T + t is token t of rank s.  A map row has W = ceil(E/8) bytes.
 */

/* Bitmap of one rank's routing: bit (e mod 8) of byte e div 8 of row t is 1
 * iff some slot j of token t selects expert e.  Masked slots (-1) set
 * nothing; ids outside [-1, E) set nothing and are counted. */
void oracle_routing_map(const int64_t *topk_idx, int64_t T, int k, int E, uint8_t *map,
                        int32_t *num_invalid)
{
    int64_t W = (E + 7) / 8;
    int32_t bad = 0;
    memset(map, 0, (size_t)(T * W));
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e == -1)
                continue;
            if (e < -1 || e >= E) {
                ++bad;
                continue;
            }
            map[t * W + e / 8] |= (uint8_t)(1u << (e % 8));
        }
    if (num_invalid)
        *num_invalid = bad;
}

static int map_bit(const uint8_t *map, int64_t W, int64_t g, int e)
{
    return (map[g * W + e / 8] >> (e % 8)) & 1;
}

/* Does global token g select any expert of rank d? */
static int routed_to_rank(const uint8_t *map, int64_t W, int64_t g, int d, int El)
{
    for (int e = d * El; e < (d + 1) * El; ++e)
        if (map_bit(map, W, g, e))
            return 1;
    return 0;
}

/*
 * Metadata preprocessing for rank `rank` from the all-gathered map
 * [G*T, W].  Rank d's receive buffer holds the tokens that select one of
 * its experts, once each, in increasing global token order.
 *
 *   sparse_to_dense [T, G]: row of rank `rank`'s token t in rank d's
 *                    receive buffer, -1 if t selects none of d's experts.
 *   num_recv:        tokens rank `rank` receives (num_tokens_for_experts).
 *   for each received row i < num_recv (global token g):
 *     local_map [i, e]   1 iff g selects local expert e (rank*El + e),
 *     recv_src [i]       g,
 *     recv_topk_idx [i]  the selected local experts in increasing order,
 *                        the first k_out of them, then -1 (selections past
 *                        k_out are counted in num_overflow),
 *   rows num_recv .. G*T-1: local_map 0, recv_src -1, recv_topk_idx -1.
 *   expert_counts [El]:  received tokens that select each local expert.
 */
void oracle_rank_layout(const uint8_t *map, int64_t T, int E, int G, int rank, int k_out,
                        int32_t *sparse_to_dense, uint8_t *local_map, int32_t *recv_src,
                        int64_t *recv_topk_idx, int32_t *expert_counts, int32_t *num_recv,
                        int32_t *num_overflow)
{
    int El = E / G;
    int64_t W = (E + 7) / 8;
    int64_t R = (int64_t)G * T;
    int32_t overflow = 0;
    for (int d = 0; d < G; ++d) {
        int32_t pos = 0;   /* rows of rank d's buffer taken so far */
        for (int64_t g = 0; g < R; ++g) {
            int hit = routed_to_rank(map, W, g, d, El);
            if (g / T == rank)
                sparse_to_dense[(g % T) * G + d] = hit ? pos : -1;
            if (hit && d == rank) {
                int n = 0;
                for (int e = 0; e < El; ++e) {
                    int b = map_bit(map, W, g, rank * El + e);
                    local_map[(int64_t)pos * El + e] = (uint8_t)b;
                    if (b) {
                        if (n < k_out)
                            recv_topk_idx[(int64_t)pos * k_out + n] = e;
                        else
                            ++overflow;
                        ++n;
                    }
                }
                for (; n < k_out; ++n)
                    recv_topk_idx[(int64_t)pos * k_out + n] = -1;
                recv_src[pos] = (int32_t)g;
            }
            if (hit)
                ++pos;
        }
        if (d == rank) {
            *num_recv = pos;
            for (int64_t i = pos; i < R; ++i) {
                for (int e = 0; e < El; ++e)
                    local_map[i * El + e] = 0;
                for (int n = 0; n < k_out; ++n)
                    recv_topk_idx[i * k_out + n] = -1;
                recv_src[i] = -1;
            }
        }
    }
    for (int e = 0; e < El; ++e) {
        int32_t c = 0;
        for (int64_t i = 0; i < *num_recv; ++i)
            c += local_map[i * El + e];
        expert_counts[e] = c;
    }
    if (num_overflow)
        *num_overflow = overflow;
}

/* Token t's weight row for rank d (k wide): the n-th selected expert of
 * rank d in increasing expert order gets the fp32 sum, in increasing j, of
 * the weights of the slots that select it (1 per slot without weights);
 * 0 past the last one. */
static void rank_weight_row(const int64_t *topk_idx, const float *topk_weights, int64_t t, int k,
                            int d, int El, float *row)
{
    for (int n = 0; n < k; ++n)
        row[n] = 0.0f;
    int n = 0;
    for (int e = d * El; e < (d + 1) * El; ++e) {
        int hit = 0;
        float s = 0.0f;
        for (int j = 0; j < k; ++j)
            if (topk_idx[t * k + j] == e) {
                s = s + (topk_weights ? topk_weights[t * k + j] : 1.0f);
                hit = 1;
            }
        if (hit) {
            if (n < k)
                row[n] = s;
            ++n;
        }
    }
}

/*
 * Dispatch of rank `rank`'s tokens, once per destination rank (NCCL EP page,
 * ncclEpDispatch high-throughput branch: the token rows and, per received
 * token, the weights of the receiving rank's experts; the receiver's
 * recv_topk_weights [N_recv, k] come from the dense-to-sparse step keyed by
 * local_expert_routing_map):
 *   dest_x[d][sparse_to_dense[t,d]] = x[t]                  (bf16 bits)
 *   dest_w[d][sparse_to_dense[t,d], n] = weight of the n-th selected expert
 *       of rank d in increasing expert order, the fp32 sum in increasing j of
 *       w[t,j] over the slots that select it (1 per slot when topk_weights
 *       is NULL); 0 for n past the last one.  Rows are k wide.
 * dest_w may be NULL, or hold NULL for a rank.
 */
void oracle_dispatch_ranked(const uint16_t *x, const int64_t *topk_idx, const float *topk_weights,
                            int64_t T, int H, int k, int E, int G,
                            const int32_t *sparse_to_dense, uint16_t *const *dest_x,
                            float *const *dest_w)
{
    int El = E / G;
    for (int64_t t = 0; t < T; ++t)
        for (int d = 0; d < G; ++d) {
            int32_t p = sparse_to_dense[t * G + d];
            if (p < 0)
                continue;
            memcpy(dest_x[d] + (int64_t)p * H, x + t * H, (size_t)H * sizeof(uint16_t));
            if (dest_w && dest_w[d])
                rank_weight_row(topk_idx, topk_weights, t, k, d, El, dest_w[d] + (int64_t)p * k);
        }
}

/*
 * Combine back to rank `rank`'s tokens (NCCL EP page, ncclEpCombine
 * high-throughput forward combine: tokens only, unweighted; each receiving
 * rank has already reduced its own experts' outputs of the token):
 *   out[t] = bf16( sum over d with sparse_to_dense[t,d] >= 0 of
 *                  src_y[d][sparse_to_dense[t,d]] ),
 * summed in fp64 in increasing d and rounded once; +0 for a token no rank
 * received.
 */
void oracle_combine_ranked(const uint16_t *const *src_y, const int32_t *sparse_to_dense, int64_t T,
                           int H, int G, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double s = 0.0;
            for (int d = 0; d < G; ++d) {
                int32_t p = sparse_to_dense[t * G + d];
                if (p >= 0)
                    s += oracle_bf16_to_double(src_y[d][(int64_t)p * H + c]);
            }
            out[t * H + c] = oracle_bf16_from_double(s);
        }
}

/*
 * Backward of the once-per-rank dispatch, for the sending rank's T tokens
 * (NCCL EP page, ncclEpCombine high-throughput branch: the backward combine
 * carries the tokens and the top-k weight gradients; each receiver turns its
 * [rows, k] weight gradients dense, keyed by local_expert_routing_map, and
 * the sender brings them back to [T, k] through its own rows of the routing
 * map; DeepEP page, "MoE Dispatch and Combine for Training/Inference with
 * ElasticBuffer": the backward of dispatch is a combine that also returns
 * the reduced weight gradients):
 *   grad_x[t] = the combine over ranks of the receivers' row gradients
 *               (oracle_combine_ranked: fp64 sum over d, one rounding)
 *   step 1, each receiver d: dense_d[row, e'] = grad_recv_w[d][row, n] for
 *           the n-th listed local expert e' = recv_topk_idx[d][row, n] >= 0
 *   step 2, the sender: grad_w[t, j] = dense_d[s2d[t, d], e - d*El] for
 *           e = topk_idx[t, j] in [0, E) and d = e / El: every slot that
 *           selected e gets the gradient of the weight sum it fed; 0 for a
 *           masked or invalid slot, or a row outside [0, rows).
 * Rows hold `rows` entries per receiver.  grad_x or grad_w may be NULL.
 */
void oracle_dispatch_ranked_backward(const uint16_t *const *grad_recv_x,
                                     const float *const *grad_recv_w,
                                     const int64_t *const *recv_topk_idx, int64_t rows,
                                     const int64_t *topk_idx, const int32_t *sparse_to_dense,
                                     int64_t T, int H, int k, int E, int G, uint16_t *grad_x,
                                     float *grad_w)
{
    if (grad_x)
        oracle_combine_ranked(grad_recv_x, sparse_to_dense, T, H, G, grad_x);
    if (!grad_w)
        return;
    int El = E / G;
    float **dense = (float **)malloc((size_t)G * sizeof(float *));
    for (int d = 0; d < G; ++d) {
        dense[d] = (float *)calloc((size_t)(rows * El > 0 ? rows * El : 1), sizeof(float));
        for (int64_t row = 0; row < rows; ++row)
            for (int n = 0; n < k; ++n) {
                int64_t e = recv_topk_idx[d][row * k + n];
                if (e >= 0 && e < El)
                    dense[d][row * El + e] = grad_recv_w[d][row * k + n];
            }
    }
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            float g = 0.0f;
            if (e >= 0 && e < E) {
                int d = (int)(e / El);
                int32_t row = sparse_to_dense[t * G + d];
                if (row >= 0 && row < rows)
                    g = dense[d][(int64_t)row * El + (e - (int64_t)d * El)];
            }
            grad_w[t * k + j] = g;
        }
    for (int d = 0; d < G; ++d)
        free(dense[d]);
    free(dense);
}

/*
 * Receive-side dispatch with the permute fused in (NeMo fused_a2a page,
 * HybridEPDispatch: fuse_permute, and the dispatched rows come out grouped
 * by local expert; NCCL EP page, sparse_to_dense_map and
 * local_expert_routing_map).  Rank `rank` takes every token it receives
 * once from the sending rank's rows and writes it to each of its
 * local-expert rows, given by `slot` [G*T, k] (the expanded layout of
 * recv_topk_idx over the E/G local experts):
 *   for received row i with g = recv_src[i] >= 0 (s = g / T, t = g % T)
 *   and j < k with slot[i, j] >= 0:
 *     recv_x[slot[i, j]] = src_x[s][t]
 *     recv_w[slot[i, j]] = the fp32 sum, in increasing j', of src_w[s][t, j']
 *         over the j' with src_idx[s][t, j'] == rank*El + recv_topk_idx[i, j]
 *         (1 per slot when src_w is NULL)
 * recv_w may be NULL.
 */
void oracle_dispatch_fused_permute(const uint16_t *const *src_x, const int64_t *const *src_idx,
                                   const float *const *src_w, int64_t T, int H, int k, int E, int G,
                                   int rank, const int32_t *recv_src, const int64_t *recv_topk_idx,
                                   const int32_t *slot, uint16_t *recv_x, float *recv_w)
{
    int El = E / G;
    for (int64_t i = 0; i < (int64_t)G * T; ++i) {
        int32_t g = recv_src[i];
        if (g < 0)
            continue;
        int s = (int)(g / T);
        int64_t t = g % T;
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[i * k + j];
            if (r < 0)
                continue;
            memcpy(recv_x + (int64_t)r * H, src_x[s] + t * H, (size_t)H * sizeof(uint16_t));
            if (!recv_w)
                continue;
            int64_t e = (int64_t)rank * El + recv_topk_idx[i * k + j];
            float sum = 0.0f;
            for (int jj = 0; jj < k; ++jj)
                if (src_idx[s][t * k + jj] == e)
                    sum = sum + (src_w && src_w[s] ? src_w[s][t * k + jj] : 1.0f);
            recv_w[r] = sum;
        }
    }
}

/*
 * The same receive-side dispatch for tokens already cast to 8 bits (NeMo
 * fused_a2a page: init_hybrid_ep_buffer's fp8_dispatch, FP8 communication
 * in the dispatch phase, and HybridEPDispatch's fuse_permute; NCCL EP page,
 * ncclEpDispatch high-throughput branch: FP8 tokens come with a 2-D fp32
 * scales tensor).  Each received token's
 * code row (H bytes) and scale row (H/128 fp32) are copied from the sending
 * rank to each of this rank's local-expert rows:
 *   recv_q[slot[i, j]] = src_q[s][t],  recv_s[slot[i, j]] = src_s[s][t]
 * and recv_w as oracle_dispatch_fused_permute (NULL: not written).
 */
void oracle_dispatch_fused_permute_prequant(const uint8_t *const *src_q,
                                            const float *const *src_s,
                                            const int64_t *const *src_idx,
                                            const float *const *src_w, int64_t T, int H, int k,
                                            int E, int G, int rank, const int32_t *recv_src,
                                            const int64_t *recv_topk_idx, const int32_t *slot,
                                            uint8_t *recv_q, float *recv_s, float *recv_w)
{
    int El = E / G;
    int nb = H / 128;
    for (int64_t i = 0; i < (int64_t)G * T; ++i) {
        int32_t g = recv_src[i];
        if (g < 0)
            continue;
        int s = (int)(g / T);
        int64_t t = g % T;
        for (int j = 0; j < k; ++j) {
            int32_t r = slot[i * k + j];
            if (r < 0)
                continue;
            for (int c = 0; c < H; ++c)
                recv_q[(int64_t)r * H + c] = src_q[s][t * H + c];
            for (int b = 0; b < nb; ++b)
                recv_s[(int64_t)r * nb + b] = src_s[s][t * nb + b];
            if (!recv_w)
                continue;
            int64_t e = (int64_t)rank * El + recv_topk_idx[i * k + j];
            float sum = 0.0f;
            for (int jj = 0; jj < k; ++jj)
                if (src_idx[s][t * k + jj] == e)
                    sum = sum + (src_w && src_w[s] ? src_w[s][t * k + jj] : 1.0f);
            recv_w[r] = sum;
        }
    }
}

/*
 * Once-per-rank dispatch of tokens already cast to 8 bits (NCCL EP page,
 * ncclEpDispatch high-throughput branch: FP8 tokens come with a 2-D fp32
 * scales tensor and travel as they are).  As oracle_dispatch_ranked, with
 * the token's code row (H bytes) and scale row (H/128 fp32) copied to each
 * destination rank that receives it:
 *   dest_q[d][p] = xq[t], dest_s[d][p] = xs[t]     (p = sparse_to_dense[t,d])
 * and the same weight rows as oracle_dispatch_ranked (dest_w may be NULL).
 */
void oracle_dispatch_ranked_prequant(const uint8_t *xq, const float *xs, const int64_t *topk_idx,
                                     const float *topk_weights, int64_t T, int H, int k, int E,
                                     int G, const int32_t *sparse_to_dense, uint8_t *const *dest_q,
                                     float *const *dest_s, float *const *dest_w)
{
    int nb = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int d = 0; d < G; ++d) {
            int32_t p = sparse_to_dense[t * G + d];
            if (p < 0)
                continue;
            memcpy(dest_q[d] + (int64_t)p * H, xq + t * H, (size_t)H);
            memcpy(dest_s[d] + (int64_t)p * nb, xs + t * nb, (size_t)nb * sizeof(float));
        }
    int El = E / G;
    for (int64_t t = 0; t < T; ++t)
        for (int d = 0; d < G; ++d) {
            int32_t p = sparse_to_dense[t * G + d];
            if (p >= 0 && dest_w && dest_w[d])
                rank_weight_row(topk_idx, topk_weights, t, k, d, El, dest_w[d] + (int64_t)p * k);
        }
}

/*
 * c_abi_demo.c -- the library driven from plain C through include/ep.h:
 * device buffers from hipMalloc, no Python and no PyTorch.
 *
 *   c_abi_demo [T H E k]        (default 1024 7168 256 8)
 *
 * Inputs are deterministic: token t selects the k distinct experts
 * (h(t) + j * (E / k)) mod E, a fixed pattern of slots is masked (-1), the
 * weights of a token's unmasked slots are equal and sum to 1, and x holds
 * bf16 values from a fixed integer hash.  The program runs ep_layout,
 * ep_dispatch (bf16) and ep_combine on the null stream, and
 * ep_layout_noalloc (no workspace) beside ep_layout, and checks what holds
 * at any size:
 *   - counts sum to the unmasked pairs, offsets are their exclusive prefix
 *     sum, slots of one expert are consecutive in pair order;
 *   - every dispatched row equals its source token, bit for bit;
 *   - combine of the dispatched rows (identity experts) with weights
 *     summing to 1 returns x (by value: a -0 element comes back +0);
 *   - ep_layout_noalloc writes the same counts, offsets, slots and sources;
 *   - the per-(token, rank) path over 4 simulated ranks (when E is a
 *     multiple of 4; rank s routes each slot to expert (e + s) mod E):
 *     ep_routing_map for every rank, ep_rank_layout for rank 0, then rank
 *     0's tokens sent once per destination rank (ep_dispatch_ranked, a host
 *     array of 4 device pointers) and gathered back (ep_combine_ranked):
 *     a token reaches rank d exactly when one of its experts is d's, every
 *     sent row equals its token, and the gather of n copies is bf16(n * x).
 * It prints one line and exits 0 when all hold, 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

#define EP_OK(call)                                                                   \
    do {                                                                              \
        ep_status_t s_ = (call);                                                              \
        if (s_ != EP_SUCCESS) {                                                       \
            fprintf(stderr, "%s: %s (%s)\n", #call, ep_status_string(s_), ep_last_error()); \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

static uint32_t hash32(uint32_t v)
{
    v ^= v >> 16;
    v *= 0x7feb352dU;
    v ^= v >> 15;
    v *= 0x846ca68bU;
    v ^= v >> 16;
    return v;
}

static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* bf16 bits of a finite float, round to nearest even */
static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)((u + 0x7FFFU + ((u >> 16) & 1U)) >> 16);
}

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    return p;
}

int main(int argc, char **argv)
{
    const int64_t T = argc > 1 ? atoll(argv[1]) : 1024;
    const int H = argc > 2 ? atoi(argv[2]) : 7168;
    const int E = argc > 3 ? atoi(argv[3]) : 256;
    const int k = argc > 4 ? atoi(argv[4]) : 8;
    if (T < 1 || H < 8 || H % 8 || E < 1 || k < 1 || k > E) {
        fprintf(stderr, "usage: c_abi_demo [T H E k], H a multiple of 8, 1 <= k <= E\n");
        return 2;
    }
    const int64_t P = T * k;
    const int stride = E / k;

    int64_t *idx = malloc(P * sizeof *idx);
    float *w = malloc(P * sizeof *w);
    uint16_t *x = malloc((size_t)T * H * sizeof *x);
    int64_t live = 0;
    for (int64_t t = 0; t < T; ++t) {
        const uint32_t h = hash32((uint32_t)t);
        int n = 0;
        for (int j = 0; j < k; ++j) {
            const int masked = (t * 7 + j) % 11 == 0;
            idx[t * k + j] = masked ? -1 : (int64_t)((h + (uint32_t)j * (uint32_t)stride) % (uint32_t)E);
            n += !masked;
        }
        for (int j = 0; j < k; ++j) w[t * k + j] = idx[t * k + j] >= 0 ? 1.0f / (float)n : 0.0f;
        live += n;
        for (int c = 0; c < H; ++c) {
            /* sign, an exponent around 1 and a 7-bit mantissa */
            const uint32_t r = hash32((uint32_t)(t * H + c) ^ 0x9e3779b9U);
            x[t * H + c] = (uint16_t)(((r & 1U) << 15) | ((0x7CU + ((r >> 1) & 3U)) << 7) | ((r >> 3) & 0x7FU));
        }
    }

    const size_t ws_bytes = ep_layout_workspace_size(T, k, E);
    int64_t *d_idx = dev_alloc(P * sizeof *d_idx);
    float *d_w = dev_alloc(P * sizeof *d_w);
    uint16_t *d_x = dev_alloc((size_t)T * H * 2);
    int32_t *d_counts = dev_alloc(E * sizeof(int32_t));
    int32_t *d_offsets = dev_alloc((E + 1) * sizeof(int32_t));
    int32_t *d_slot = dev_alloc(P * sizeof(int32_t));
    int32_t *d_src = dev_alloc(P * sizeof(int32_t));
    int32_t *d_inval = dev_alloc(sizeof(int32_t));
    void *d_ws = dev_alloc(ws_bytes);
    uint16_t *d_recv = dev_alloc((size_t)P * H * 2);
    float *d_recv_w = dev_alloc(P * sizeof(float));
    uint16_t *d_out = dev_alloc((size_t)T * H * 2);
    int32_t *d_counts2 = dev_alloc(E * sizeof(int32_t));
    int32_t *d_offsets2 = dev_alloc((E + 1) * sizeof(int32_t));
    int32_t *d_slot2 = dev_alloc(P * sizeof(int32_t));
    int32_t *d_src2 = dev_alloc(P * sizeof(int32_t));
    HIP_OK(hipMemcpy(d_idx, idx, P * sizeof *idx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, P * sizeof *w, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, (size_t)T * H * 2, hipMemcpyHostToDevice));

    EP_OK(ep_layout(d_idx, T, k, E, d_counts, d_offsets, d_slot, d_src, d_inval, d_ws, ws_bytes,
                    NULL));
    EP_OK(ep_dispatch(d_x, T, H, k, d_slot, d_w, EP_OUT_BF16, d_recv, NULL, d_recv_w, NULL));
    EP_OK(ep_combine(d_recv, d_slot, d_w, T, H, k, d_out, NULL));
    EP_OK(ep_layout_noalloc(d_idx, T, k, E, d_counts2, d_offsets2, d_slot2, d_src2, NULL, NULL));
    HIP_OK(hipDeviceSynchronize());

    int32_t *counts = malloc(E * sizeof *counts);
    int32_t *offsets = malloc((E + 1) * sizeof *offsets);
    int32_t *slot = malloc(P * sizeof *slot);
    uint16_t *recv = malloc((size_t)P * H * 2);
    uint16_t *out = malloc((size_t)T * H * 2);
    int32_t inval = -1;
    HIP_OK(hipMemcpy(counts, d_counts, E * sizeof *counts, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(offsets, d_offsets, (E + 1) * sizeof *offsets, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(slot, d_slot, P * sizeof *slot, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv, d_recv, (size_t)P * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out, d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&inval, d_inval, sizeof inval, hipMemcpyDeviceToHost));
    int32_t *counts2 = malloc(E * sizeof *counts2);
    int32_t *offsets2 = malloc((E + 1) * sizeof *offsets2);
    int32_t *slot2 = malloc(P * sizeof *slot2);
    int32_t *src = malloc(P * sizeof *src);
    int32_t *src2 = malloc(P * sizeof *src2);
    HIP_OK(hipMemcpy(counts2, d_counts2, E * sizeof *counts2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(offsets2, d_offsets2, (E + 1) * sizeof *offsets2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(slot2, d_slot2, P * sizeof *slot2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(src, d_src, P * sizeof *src, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(src2, d_src2, P * sizeof *src2, hipMemcpyDeviceToHost));

    /* layout: counts, exclusive offsets, no invalid entries */
    int layout_ok = inval == 0;
    int64_t sum = 0;
    for (int e = 0; e < E; ++e) {
        layout_ok = layout_ok && offsets[e] == sum;
        sum += counts[e];
    }
    layout_ok = layout_ok && sum == live && offsets[E] == live;
    /* slots consecutive per expert in pair order; each row equals its token */
    int rows_ok = 1;
    int32_t *next = malloc(E * sizeof *next);
    memcpy(next, offsets, E * sizeof *next);
    for (int64_t i = 0; i < P; ++i) {
        const int64_t e = idx[i];
        if (e < 0) {
            layout_ok = layout_ok && slot[i] == -1;
            continue;
        }
        if (slot[i] != next[e]++) {
            layout_ok = 0;
            break;
        }
        rows_ok = rows_ok &&
                  memcmp(recv + (size_t)slot[i] * H, x + (size_t)(i / k) * H, (size_t)H * 2) == 0;
    }
    /* combine returns x by value (a token with every slot masked gives 0) */
    int64_t bad = 0;
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int j = 0; j < k; ++j) any |= idx[t * k + j] >= 0;
        for (int c = 0; c < H; ++c) {
            const float want = any ? bf16_value(x[t * H + c]) : 0.0f;
            bad += bf16_value(out[t * H + c]) != want;
        }
    }
    /* the no-allocation layout: the same outputs (src over the routed rows) */
    const int noalloc_ok = memcmp(counts, counts2, E * sizeof *counts) == 0 &&
                           memcmp(offsets, offsets2, (E + 1) * sizeof *offsets) == 0 &&
                           memcmp(slot, slot2, P * sizeof *slot) == 0 &&
                           memcmp(src, src2, (size_t)live * sizeof *src) == 0;

    /* the per-(token, rank) path, rank 0 of 4 */
    enum { G = 4 };
    const char *ranked = "skipped (E not a multiple of 4)";
    int ranked_ok = 1;
    if (E % G == 0) {
        const int W = (E + 7) / 8, El = E / G;
        uint8_t *d_gmap = dev_alloc((size_t)G * T * W);
        int64_t *idx_s = malloc(P * sizeof *idx_s);
        int64_t *d_idx_s = dev_alloc(P * sizeof *d_idx_s);
        for (int r = 0; r < G; ++r) {
            for (int64_t i = 0; i < P; ++i) idx_s[i] = idx[i] < 0 ? -1 : (idx[i] + r) % E;
            HIP_OK(hipMemcpy(d_idx_s, idx_s, P * sizeof *idx_s, hipMemcpyHostToDevice));
            EP_OK(ep_routing_map(d_idx_s, T, k, E, d_gmap + (size_t)r * T * W, NULL, NULL));
            HIP_OK(hipDeviceSynchronize());
        }
        const size_t rws_bytes = ep_rank_layout_workspace_size(T, E, G);
        int32_t *d_s2d = dev_alloc((size_t)T * G * sizeof(int32_t));
        uint8_t *d_lm = dev_alloc((size_t)G * T * El);
        int32_t *d_rsrc = dev_alloc((size_t)G * T * sizeof(int32_t));
        int64_t *d_rti = dev_alloc((size_t)G * T * k * sizeof(int64_t));
        int32_t *d_ecnt = dev_alloc(El * sizeof(int32_t));
        int32_t *d_nrecv = dev_alloc(sizeof(int32_t));
        int32_t *d_novf = dev_alloc(sizeof(int32_t));
        void *d_rws = dev_alloc(rws_bytes);
        EP_OK(ep_rank_layout(d_gmap, T, E, G, 0, k, d_s2d, d_lm, d_rsrc, d_rti, d_ecnt, d_nrecv,
                             d_novf, d_rws, rws_bytes, NULL));
        /* rank 0 sends first, so its rows in every buffer are below T */
        void *dest[G];
        for (int d = 0; d < G; ++d) dest[d] = dev_alloc((size_t)T * H * 2);
        uint16_t *d_out_r = dev_alloc((size_t)T * H * 2);
        EP_OK(ep_dispatch_ranked(d_x, d_idx, d_w, T, H, k, E, G, d_s2d, dest, NULL, T, NULL));
        EP_OK(ep_combine_ranked((const void *const *)dest, T, d_s2d, T, H, G, d_out_r, NULL));
        HIP_OK(hipDeviceSynchronize());
        int32_t *s2d = malloc((size_t)T * G * sizeof *s2d);
        uint16_t *rows = malloc((size_t)T * H * 2);
        HIP_OK(hipMemcpy(s2d, d_s2d, (size_t)T * G * sizeof *s2d, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(out, d_out_r, (size_t)T * H * 2, hipMemcpyDeviceToHost));
        for (int d = 0; d < G && ranked_ok; ++d) {
            HIP_OK(hipMemcpy(rows, dest[d], (size_t)T * H * 2, hipMemcpyDeviceToHost));
            for (int64_t t = 0; t < T && ranked_ok; ++t) {
                int reaches = 0;
                for (int j = 0; j < k; ++j)
                    reaches |= idx[t * k + j] >= (int64_t)d * El && idx[t * k + j] < (int64_t)(d + 1) * El;
                const int32_t r = s2d[t * G + d];
                ranked_ok = (r >= 0) == reaches && r < T &&
                            (r < 0 || memcmp(rows + (size_t)r * H, x + (size_t)t * H, (size_t)H * 2) == 0);
            }
        }
        for (int64_t t = 0; t < T && ranked_ok; ++t) {
            int n = 0;
            for (int d = 0; d < G; ++d) n += s2d[t * G + d] >= 0;
            for (int c = 0; c < H && ranked_ok; ++c) {
                const uint16_t want = n ? bf16_rne((float)n * bf16_value(x[t * H + c])) : 0;
                ranked_ok = out[t * H + c] == want;
            }
        }
        ranked = ranked_ok ? "ok" : "WRONG";
    }
    const int ok = layout_ok && rows_ok && bad == 0 && noalloc_ok && ranked_ok;

    printf("c_abi_demo T=%lld H=%d E=%d k=%d: %lld of %lld pairs routed; layout %s, rows %s, "
           "combine %s (%lld elements off), noalloc %s, ranked %s\n",
           (long long)T, H, E, k, (long long)live, (long long)P, layout_ok ? "ok" : "WRONG",
           rows_ok ? "ok" : "WRONG", bad == 0 ? "ok" : "WRONG", (long long)bad,
           noalloc_ok ? "ok" : "WRONG", ranked);
    return ok ? 0 : 1;
}

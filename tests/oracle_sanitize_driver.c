/*
 * Drives every function of oracle/ep_oracle.c on small seeded inputs, with
 * invariant checks, for a build with -fsanitize=address,undefined: a check
 * of the oracle's memory safety and defined behaviour, run on the CPU by
 * tests/test_oracle_sanitize.py.  Test infrastructure only.
 *
 * Checks: codec round trips over every code; layout invariants (counts,
 * exclusive offsets, slots a bijection onto the rows in stable order, src);
 * dispatch rows equal their token's row (bf16), equal across a token's
 * slots (8-bit casts); unit-weight combine of identity experts returns x;
 * the per-rank path's receive rows and combine.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t b);
uint16_t oracle_bf16_from_double(double d);
double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float v);
double oracle_e5m2_decode(uint8_t c);
uint8_t oracle_e5m2_encode(float v);
void oracle_layout_ex(const int64_t *topk_idx, int64_t T, int k, int E, int alignment,
                      int64_t expert_capacity, int32_t *counts, int32_t *offsets,
                      int32_t *slot, int32_t *src, int32_t *num_invalid, int32_t *num_dropped);
void oracle_layout(const int64_t *topk_idx, int64_t T, int k, int E, int32_t *counts,
                   int32_t *offsets, int32_t *slot, int32_t *src, int32_t *num_invalid);
void oracle_dispatch_bf16(const uint16_t *x, int64_t T, int H, int k, const int32_t *slot,
                          const float *topk_weights, uint16_t *recv_x, float *recv_w);
void oracle_dispatch_fp8(const uint16_t *x, int64_t T, int H, int k, const int32_t *slot,
                         const float *topk_weights, uint8_t *recv_q, float *recv_scales,
                         float *recv_w);
void oracle_combine(const uint16_t *y, const int32_t *slot, const float *topk_weights, int64_t T,
                    int H, int k, uint16_t *out);
void oracle_combine_backward(const uint16_t *g, const uint16_t *y, const int32_t *slot,
                             const float *topk_weights, int64_t T, int H, int k, uint16_t *grad_y,
                             float *grad_w);
void oracle_dispatch_backward(const uint16_t *grad_recv, const float *grad_recv_w,
                              const int32_t *slot, int64_t T, int H, int k, uint16_t *grad_x,
                              float *grad_w);
void oracle_dispatch_quant(const uint16_t *x, int64_t T, int H, int k, const int32_t *slot,
                           const float *topk_weights, int format, int scale_mode, uint8_t *recv_q,
                           void *recv_scales, float *recv_w);
void oracle_dispatch_prequant(const uint8_t *xq, const float *xs, int64_t T, int H, int k,
                              const int32_t *slot, const float *topk_weights, uint8_t *recv_q,
                              float *recv_s, float *recv_w);
void oracle_routing_map(const int64_t *topk_idx, int64_t T, int k, int E, uint8_t *map,
                        int32_t *num_invalid);
void oracle_rank_layout(const uint8_t *map, int64_t T, int E, int G, int rank, int k_out,
                        int32_t *sparse_to_dense, uint8_t *local_map, int32_t *recv_src,
                        int64_t *recv_topk_idx, int32_t *expert_counts, int32_t *num_recv,
                        int32_t *num_overflow);
void oracle_dispatch_ranked(const uint16_t *x, const int64_t *topk_idx, const float *topk_weights,
                            int64_t T, int H, int k, int E, int G, const int32_t *sparse_to_dense,
                            uint16_t *const *dest_x, float *const *dest_w);
void oracle_combine_ranked(const uint16_t *const *src_y, const int32_t *sparse_to_dense, int64_t T,
                           int H, int G, uint16_t *out);
void oracle_dispatch_fused_permute(const uint16_t *const *src_x, const int64_t *const *src_idx,
                                   const float *const *src_w, int64_t T, int H, int k, int E, int G,
                                   int rank, const int32_t *recv_src, const int64_t *recv_topk_idx,
                                   const int32_t *slot, uint16_t *recv_x, float *recv_w);
void oracle_dispatch_fused_permute_prequant(const uint8_t *const *src_q, const float *const *src_s,
                                            const int64_t *const *src_idx,
                                            const float *const *src_w, int64_t T, int H, int k,
                                            int E, int G, int rank, const int32_t *recv_src,
                                            const int64_t *recv_topk_idx, const int32_t *slot,
                                            uint8_t *recv_q, float *recv_s, float *recv_w);
void oracle_dispatch_ranked_prequant(const uint8_t *xq, const float *xs, const int64_t *topk_idx,
                                     const float *topk_weights, int64_t T, int H, int k, int E,
                                     int G, const int32_t *sparse_to_dense, uint8_t *const *dest_q,
                                     float *const *dest_s, float *const *dest_w);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}

#define CHECK(c)                                                                 \
    do {                                                                         \
        if (!(c)) {                                                              \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);      \
            exit(1);                                                             \
        }                                                                        \
    } while (0)

static void *xalloc(size_t n)
{
    void *p = calloc(n ? n : 1, 1);
    CHECK(p != NULL);
    return p;
}

/* a finite bf16 value of moderate size with random sign */
static uint16_t rnd_bf16(void)
{
    uint32_t e = 112 + rnd() % 24, m = rnd() & 0x7F, s = rnd() & 1;
    return (uint16_t)(s << 15 | e << 7 | m);
}

static void check_layout(const int64_t *idx, int T, int k, int E, const int32_t *counts,
                         const int32_t *offsets, const int32_t *slot, const int32_t *src)
{
    int32_t valid = 0;
    for (int i = 0; i < T * k; ++i)
        valid += idx[i] >= 0 && idx[i] < E;
    CHECK(offsets[0] == 0);
    for (int e = 0; e < E; ++e)
        CHECK(offsets[e + 1] == offsets[e] + counts[e]);
    CHECK(offsets[E] == valid);
    int32_t *seen = xalloc((size_t)(valid + 1) * sizeof(int32_t));
    int32_t *last = xalloc((size_t)E * sizeof(int32_t));
    for (int e = 0; e < E; ++e)
        last[e] = offsets[e] - 1;
    for (int i = 0; i < T * k; ++i) {
        int64_t e = idx[i];
        if (e < 0 || e >= E) {
            CHECK(slot[i] == -1);
            continue;
        }
        int32_t r = slot[i];
        CHECK(r >= offsets[e] && r < offsets[e + 1]);
        CHECK(r == last[e] + 1);             /* stable: rows in flat pair order */
        last[e] = r;
        CHECK(!seen[r]);
        seen[r] = 1;
        CHECK(src[r] == i / k);
    }
    free(seen);
    free(last);
}

int main(void)
{
    /* codecs: every code */
    for (uint32_t b = 0; b < 65536; ++b) {
        double d = oracle_bf16_to_double((uint16_t)b);
        if (!isnan(d))
            CHECK(oracle_bf16_from_double(d) == b);
    }
    for (uint32_t c = 0; c < 256; ++c) {
        double v = oracle_e4m3_decode((uint8_t)c);
        if (!isnan(v))
            CHECK(oracle_e4m3_encode((float)v) == c);
        double u = oracle_e5m2_decode((uint8_t)c);
        if (isfinite(u))
            CHECK(oracle_e5m2_encode((float)u) == c);
    }

    for (int cs = 0; cs < 150; ++cs) {
        int T = 1 + (int)(rnd() % 40), k = 1 + (int)(rnd() % 6), E = 1 + (int)(rnd() % 10);
        int H = 128 * (1 + (int)(rnd() % 3)), P = T * k, nb = H / 128;
        int64_t *idx = xalloc((size_t)P * sizeof(int64_t));
        for (int i = 0; i < P; ++i) {
            uint32_t r = rnd() % 100;
            idx[i] = r < 10 ? -1 : r < 14 ? (r & 1 ? E + 3 : -5) : (int64_t)(rnd() % (uint32_t)E);
        }
        uint16_t *x = xalloc((size_t)T * H * 2);
        float *w = xalloc((size_t)P * 4);
        for (int i = 0; i < T * H; ++i)
            x[i] = rnd_bf16();
        for (int i = 0; i < P; ++i)
            w[i] = (float)(rnd() % 1000) / 1000.0f;

        int32_t *counts = xalloc((size_t)E * 4), *offsets = xalloc((size_t)(E + 1) * 4);
        int32_t *slot = xalloc((size_t)P * 4), *src = xalloc((size_t)P * 4), inval = 0, drop = 0;
        oracle_layout(idx, T, k, E, counts, offsets, slot, src, &inval);
        check_layout(idx, T, k, E, counts, offsets, slot, src);
        int N = offsets[E];

        /* aligned and fixed-stride placements */
        int A = 1 + (int)(rnd() % 4), cap = (rnd() & 1) ? A * (1 + (int)(rnd() % 3)) : 0;
        int rows_ex = cap ? E * cap : P + E * (A - 1);
        int32_t *cnt2 = xalloc((size_t)E * 4), *off2 = xalloc((size_t)(E + 1) * 4);
        int32_t *slot2 = xalloc((size_t)P * 4), *src2 = xalloc((size_t)(rows_ex + 1) * 4);
        oracle_layout_ex(idx, T, k, E, A, cap, cnt2, off2, slot2, src2, &inval, &drop);
        for (int i = 0; i < P; ++i)
            CHECK(slot2[i] < rows_ex);
        for (int e = 0; e < E; ++e)
            CHECK(off2[e] % A == 0 || cap);

        /* dispatches */
        uint16_t *recv = xalloc((size_t)P * H * 2);
        float *rw = xalloc((size_t)P * 4);
        oracle_dispatch_bf16(x, T, H, k, slot, w, recv, rw);
        for (int i = 0; i < P; ++i)
            if (slot[i] >= 0) {
                CHECK(!memcmp(recv + (size_t)slot[i] * H, x + (size_t)(i / k) * H, (size_t)H * 2));
                CHECK(rw[slot[i]] == w[i]);
            }
        uint8_t *q = xalloc((size_t)P * H);
        float *sc = xalloc((size_t)P * nb * 4);
        oracle_dispatch_fp8(x, T, H, k, slot, w, q, sc, rw);
        for (int fmt = 0; fmt < 2; ++fmt)
            for (int mode = 0; mode < 3; ++mode) {
                oracle_dispatch_quant(x, T, H, k, slot, w, fmt, mode, q, sc, rw);
                for (int t = 0; t < T; ++t)
                    for (int j = 1; j < k; ++j) {
                        int32_t a = slot[t * k], b = slot[t * k + j];
                        if (a >= 0 && b >= 0)
                            CHECK(!memcmp(q + (size_t)a * H, q + (size_t)b * H, (size_t)H));
                    }
            }
        uint8_t *xq = xalloc((size_t)T * H);
        float *xs = xalloc((size_t)T * nb * 4);
        for (int i = 0; i < T * H; ++i)
            xq[i] = (uint8_t)rnd();
        oracle_dispatch_prequant(xq, xs, T, H, k, slot, w, q, sc, rw);

        /* combine: unit weights over identity experts count each slot once */
        uint16_t *out = xalloc((size_t)T * H * 2);
        oracle_combine(recv, slot, NULL, T, H, k, out);
        for (int t = 0; t < T; ++t) {
            int n = 0;
            for (int j = 0; j < k; ++j)
                n += slot[t * k + j] >= 0;
            for (int c = 0; c < H; ++c) {
                double want = n * oracle_bf16_to_double(x[(size_t)t * H + c]);
                double got = oracle_bf16_to_double(out[(size_t)t * H + c]);
                CHECK(fabs(got - want) <= fabs(want) * 0x1p-8);
            }
        }
        oracle_combine(recv, slot, w, T, H, k, out);
        uint16_t *gy = xalloc((size_t)P * H * 2);
        float *gw = xalloc((size_t)P * 4);
        oracle_combine_backward(x, recv, slot, w, T, H, k, gy, gw);
        oracle_dispatch_backward(recv, rw, slot, T, H, k, out, gw);

        free(idx); free(x); free(w); free(counts); free(offsets); free(slot); free(src);
        free(cnt2); free(off2); free(slot2); free(src2); free(recv); free(rw); free(q); free(sc);
        free(xq); free(xs); free(out); free(gy); free(gw);
    }

    /* the per-(token, rank) path: G ranks of T tokens, El experts each */
    for (int cs = 0; cs < 60; ++cs) {
        int G = 1 + (int)(rnd() % 3), El = 1 + (int)(rnd() % 4), E = G * El;
        int T = 1 + (int)(rnd() % 20), k = 1 + (int)(rnd() % 4), H = 128, W = (E + 7) / 8;
        int R = G * T;
        int64_t *idx = xalloc((size_t)R * k * 8);
        for (int i = 0; i < R * k; ++i)
            idx[i] = (rnd() % 8 == 0) ? -1 : (int64_t)(rnd() % (uint32_t)E);
        uint8_t *map = xalloc((size_t)R * W);
        int32_t inval = 0;
        oracle_routing_map(idx, R, k, E, map, &inval);
        uint16_t **xs_r = xalloc((size_t)G * sizeof(void *));
        float **ws_r = xalloc((size_t)G * sizeof(void *));
        for (int s = 0; s < G; ++s) {
            xs_r[s] = xalloc((size_t)T * H * 2);
            ws_r[s] = xalloc((size_t)T * k * 4);
            for (int i = 0; i < T * H; ++i)
                xs_r[s][i] = rnd_bf16();
            for (int i = 0; i < T * k; ++i)
                ws_r[s][i] = (float)(rnd() % 100) / 100.0f;
        }
        int rank = (int)(rnd() % (uint32_t)G);
        int32_t *s2d = xalloc((size_t)T * G * 4), *rsrc = xalloc((size_t)R * 4);
        uint8_t *lmap = xalloc((size_t)R * El);
        int64_t *rtopk = xalloc((size_t)R * k * 8);
        int32_t *ecnt = xalloc((size_t)El * 4), nrecv = 0, novf = 0;
        oracle_rank_layout(map, T, E, G, rank, k, s2d, lmap, rsrc, rtopk, ecnt, &nrecv, &novf);
        CHECK(nrecv >= 0 && nrecv <= R);
        for (int i = nrecv; i < R; ++i)
            CHECK(rsrc[i] == -1);

        uint16_t **dest = xalloc((size_t)G * sizeof(void *));
        float **destw = xalloc((size_t)G * sizeof(void *));
        uint8_t **destq = xalloc((size_t)G * sizeof(void *));
        float **dests = xalloc((size_t)G * sizeof(void *));
        for (int d = 0; d < G; ++d) {
            dest[d] = xalloc((size_t)R * H * 2);
            destw[d] = xalloc((size_t)R * k * 4);
            destq[d] = xalloc((size_t)R * H);
            dests[d] = xalloc((size_t)R * 4);
        }
        const int64_t *my_idx = idx + (size_t)rank * T * k;
        oracle_dispatch_ranked(xs_r[rank], my_idx, ws_r[rank], T, H, k, E, G, s2d, dest, destw);
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < G; ++d)
                if (s2d[t * G + d] >= 0)
                    CHECK(!memcmp(dest[d] + (size_t)s2d[t * G + d] * H, xs_r[rank] + (size_t)t * H,
                                  (size_t)H * 2));
        uint16_t *out = xalloc((size_t)T * H * 2);
        oracle_combine_ranked((const uint16_t *const *)dest, s2d, T, H, G, out);
        uint8_t *xq = xalloc((size_t)T * H);
        float *xsc = xalloc((size_t)T * 4);
        oracle_dispatch_ranked_prequant(xq, xsc, my_idx, ws_r[rank], T, H, k, E, G, s2d, destq,
                                        dests, destw);

        /* fused permute on the receiving side of `rank` */
        const int64_t **src_idx = xalloc((size_t)G * sizeof(void *));
        for (int s = 0; s < G; ++s)
            src_idx[s] = idx + (size_t)s * T * k;
        int32_t *cnt = xalloc((size_t)El * 4), *off = xalloc((size_t)(El + 1) * 4);
        int32_t *pslot = xalloc((size_t)R * k * 4), *psrc = xalloc((size_t)R * k * 4);
        oracle_layout(rtopk, R, k, El, cnt, off, pslot, psrc, &inval);
        uint16_t *px = xalloc((size_t)R * k * H * 2);
        float *pw = xalloc((size_t)R * k * 4);
        oracle_dispatch_fused_permute((const uint16_t *const *)xs_r, src_idx,
                                      (const float *const *)ws_r, T, H, k, E, G, rank, rsrc, rtopk,
                                      pslot, px, pw);
        /* and its 8-bit form: every rank sends the same code and scale rows */
        const uint8_t **sq = xalloc((size_t)G * sizeof(void *));
        const float **ssc = xalloc((size_t)G * sizeof(void *));
        for (int s = 0; s < G; ++s) {
            sq[s] = xq;
            ssc[s] = xsc;
        }
        uint8_t *pq = xalloc((size_t)R * k * H);
        float *ps = xalloc((size_t)R * k * 4);
        oracle_dispatch_fused_permute_prequant(sq, ssc, src_idx, (const float *const *)ws_r, T, H, k,
                                               E, G, rank, rsrc, rtopk, pslot, pq, ps, pw);
        free(sq); free(ssc); free(pq); free(ps);

        for (int s = 0; s < G; ++s) {
            free(xs_r[s]);
            free(ws_r[s]);
        }
        for (int d = 0; d < G; ++d) {
            free(dest[d]); free(destw[d]); free(destq[d]); free(dests[d]);
        }
        free(idx); free(map); free(xs_r); free(ws_r); free(s2d); free(rsrc); free(lmap); free(rtopk);
        free(ecnt); free(dest); free(destw); free(destq); free(dests); free(out); free(xq); free(xsc);
        free(src_idx); free(cnt); free(off); free(pslot); free(psrc); free(px); free(pw);
    }
    printf("oracle sanitize driver: ok\n");
    return 0;
}

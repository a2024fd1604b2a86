/*
 * ep.h -- C ABI of the MoE token layout / dispatch / combine library
 * (libep.so, HIP kernels for AMD Instinct MI355X, gfx950).
 *
 * One device's share of expert-parallel token routing, with every buffer in
 * that device's memory:
 *
 *   ep_layout    topk_idx [T,k]  ->  per-expert counts, exclusive offsets,
 *                stable destination row ("slot") of every (token, k) pair,
 *                and the source token of every destination row;
 *   ep_dispatch  copy (bf16) or cast (OCP E4M3 with one fp32 scale per 128
 *                channels) every token row into the expert-grouped buffer;
 *   ep_combine   gather the expert-output rows back and reduce them per
 *                token, weighted by topk_weights, in fp32, in top-k order.
 *
 * Around them: ep_layout_ex (aligned segments, fixed capacity),
 * ep_layout_noalloc (no workspace argument), ep_dispatch_ex and the
 * pre-quantized / column-major-scale forms (8-bit variants), the two
 * backward passes, and the per-(token, rank) path (ep_routing_map,
 * ep_rank_layout, ep_dispatch_ranked and its 8-bit forms, the fused
 * permutes, ep_combine_ranked, ep_dispatch_ranked_backward), each declared
 * below with the passage it follows.
 *
 * The operations follow the pages' problem statement:
 *   - NCCL EP (nccl_ep.cc): ncclEpCreateHandle (topk_idx is a 2-D int64
 *     tensor; "Step 3" metadata preprocessing gives per-expert counts),
 *     ncclEpDispatch (bf16 tokens with hidden a multiple of 8 elements; fp8
 *     scales of hidden/128 fp32 per token), ncclEpCombine (low-latency
 *     branch: reduction weighted by topk_weights [T,k] fp32; high-throughput
 *     forward: unweighted);
 *   - DeepEP ElasticBuffer dispatch() / combine() and EPHandle's prefix sums
 *     ("Prefix Sum Interpretation for Expert Token Counts": expert i owns
 *     rows [psum[i-1], psum[i]) of the expanded, one-slot-per-token-per-
 *     expert receive buffer);
 *   - NeMo fused_a2a HybridEPDispatch: topk_idx uses -1 for an unused slot;
 *     the dispatched rows are grouped by expert.
 *
 * Conventions shared by every call
 *   - All array arguments are device pointers (memory the GPU can read and
 *     write: hipMalloc'd, or torch CUDA tensors).  The caller owns them; the
 *     library never frees, keeps or allocates memory and holds no state
 *     between calls (apart from ep_layout_noalloc's fixed per-device
 *     scratch), so the layout outputs themselves are the "handle" that
 *     dispatch and combine take.
 *   - bf16 / fp8 / fp32 row buffers must be 16-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream).  Arguments are checked on the host before anything is
 *     launched; a failed check returns EP_INVALID_ARGUMENT (or
 *     EP_UNSUPPORTED) and launches nothing.  A HIP launch error returns
 *     EP_RUNTIME_ERROR.  The library never aborts or exits.
 *   - Data-dependent problems cannot be reported synchronously: a topk_idx
 *     entry outside [-1, E) is treated as masked and counted in
 *     *num_invalid.
 *   - ep_last_error() returns a message for the last failed call on the
 *     calling thread.
 */
#ifndef EP_H_
#define EP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_SUCCESS = 0,
    EP_INVALID_ARGUMENT = 1,
    EP_UNSUPPORTED = 2,
    EP_RUNTIME_ERROR = 3
} ep_status_t;

typedef enum {
    EP_OUT_BF16 = 0,      /* recv_x is bf16 [rows, hidden]                  */
    EP_OUT_FP8_E4M3 = 1,  /* recv_x is OCP E4M3 bytes [rows, hidden] plus
                             recv_scales [rows, hidden/128]                 */
    EP_OUT_FP8_E5M2 = 2   /* recv_x is OCP E5M2 bytes, likewise             */
} ep_out_dtype_t;

typedef enum {
    EP_SCALE_FP32 = 0,      /* fp32 scale = amax / max_finite                 */
    EP_SCALE_FP32_POW2 = 1, /* fp32 scale = 2^e, e the smallest integer with
                               2^e >= amax / max_finite (rounded-up scale)   */
    EP_SCALE_UE8M0 = 2      /* the same 2^e stored as one UE8M0 byte e + 127,
                               e clamped to -127                             */
} ep_scale_format_t;

/* Limits checked by every call. */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 64
#define EP_MAX_HIDDEN 65536
#define EP_MAX_ALIGNMENT 4096
#define EP_MAX_RANKS 64

/* Library version, (major << 16) | minor. */
int ep_version(void);

/* Static text for a status code. */
const char *ep_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char *ep_last_error(void);

/*
 * Bytes of device scratch ep_layout needs for this shape (a multiple of
 * 256).  Pure host arithmetic; returns 0 for an invalid shape.
 */
size_t ep_layout_workspace_size(int64_t num_tokens, int num_topk, int num_experts);

/*
 * ep_layout -- routing layout of one device's tokens.
 *
 * Passages: NCCL EP page, nccl_ep.cc, ncclEpCreateHandle (int64 topk_idx
 * [T,k]; "Step 3" preprocessing yields per-expert token counts and the
 * received-token total); DeepEP page, dispatch() do_expand and "Prefix Sum
 * Interpretation for Expert Token Counts"; NeMo fused_a2a page,
 * HybridEPDispatch topk_idx with -1 for unused slots.
 *
 * In:  topk_idx     int64 [num_tokens, num_topk] row-major; -1 = masked,
 *                   anything else outside [0, num_experts) is invalid and
 *                   treated as masked.
 * Out: counts       int32 [num_experts]: unmasked pairs per expert.
 *      offsets      int32 [num_experts + 1]: exclusive prefix sum of counts;
 *                   offsets[E] = N, the number of dispatched rows.
 *      slot         int32 [num_tokens * num_topk]: destination row of pair
 *                   (t, j) at index t*k + j, or -1 if masked.  Rows of one
 *                   expert are handed out in increasing t*k + j order
 *                   (a stable counting sort), so the result is
 *                   deterministic.
 *      src          int32 [num_tokens * num_topk] or NULL: src[r] = source
 *                   token of row r for r < N; entries >= N are not written.
 *                   (With ep_layout_ex, src needs ep_layout_max_rows rows.)
 *      num_invalid  int32 [1] or NULL: number of invalid entries.
 * Scratch: workspace of at least ep_layout_workspace_size(...) bytes,
 *      256-byte aligned; contents need not be initialised and are
 *      clobbered.
 * num_tokens may be 0 (then counts and offsets are zero-filled).
 * Requires num_tokens * num_topk < 2^31, 1 <= num_topk <= EP_MAX_TOPK,
 * 1 <= num_experts <= EP_MAX_EXPERTS.
 */
ep_status_t ep_layout(const int64_t *topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                      int32_t *counts, int32_t *offsets, int32_t *slot, int32_t *src,
                      int32_t *num_invalid, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ep_layout_noalloc -- ep_layout for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc): the scratch is a fixed array the library holds on each
 * device (EP_LAYOUT_NOALLOC_SCRATCH_BYTES, its size, is enough for every
 * shape ep_layout accepts: 256 chunks of EP_MAX_EXPERTS counts), so the
 * call takes no workspace and allocates nothing.  The first call on a
 * device looks up that device's array (hipGetSymbolAddress, with the
 * device current); make it once before graph capture if the capture must
 * hold launches only.
 *
 * Arguments, outputs and errors as ep_layout, minus the workspace; a shape
 * whose scratch need exceeds the array returns EP_UNSUPPORTED (none that
 * ep_layout accepts does).  Nothing in the scratch needs clearing: the
 * first launch writes every entry the second reads.  All calls on one
 * device share its array: calls that may overlap on one device (on
 * different streams without ordering between them) race and must not be
 * made; calls ordered on one stream are safe.
 */
#define EP_LAYOUT_NOALLOC_SCRATCH_BYTES ((size_t)(256 * 1024 + 256) * 4)
ep_status_t ep_layout_noalloc(const int64_t *topk_idx, int64_t num_tokens, int num_topk,
                              int num_experts, int32_t *counts, int32_t *offsets, int32_t *slot,
                              int32_t *src, int32_t *num_invalid, void *stream);

/*
 * ep_layout_ex -- ep_layout with the segment placements the pages' expanded
 * layouts offer.  ep_layout is ep_layout_ex(alignment 1, capacity 0).
 *
 * Passages: DeepEP page, dispatch() expert_alignment and "Prefix Sum
 * Interpretation for Expert Token Counts" (in expand mode expert i's rows
 * start at align(psum[i-1], expert_alignment) and end at psum[i]); NeMo
 * fused_a2a page, HybridEPDispatch pad_multiple; NCCL EP page,
 * ncclEpDispatch low-latency branch (recv_x [num_local_experts, capacity,
 * hidden] with a per-expert receive count).
 *
 *   alignment        1..EP_MAX_ALIGNMENT.  With expert_capacity == 0 the
 *                    segments are packed: expert e starts at
 *                    offsets[e] = sum_{e'<e} round_up(counts[e'], alignment),
 *                    and offsets[E] is the padded total; DeepEP's
 *                    psum[e] = offsets[e] + counts[e].
 *   expert_capacity  0, or a positive multiple of alignment: fixed stride,
 *                    expert e owns rows [e*cap, (e+1)*cap), offsets[e] =
 *                    e*cap, offsets[E] = E*cap.  Pairs whose rank within
 *                    their expert (in flat order) reaches cap are dropped:
 *                    slot -1, counted in *num_dropped; counts[e] is the
 *                    number of rows placed, at most cap.
 *   num_dropped      int32 [1] or NULL.
 * Padding rows are never written by ep_layout (src) or by ep_dispatch.
 * A receive buffer of ep_layout_max_rows(...) rows is always enough.
 * Other arguments, errors and requirements as ep_layout; additionally the
 * layout's row count bound must be below 2^31 (else EP_UNSUPPORTED).
 */
ep_status_t ep_layout_ex(const int64_t *topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                         int alignment, int64_t expert_capacity, int32_t *counts, int32_t *offsets,
                         int32_t *slot, int32_t *src, int32_t *num_invalid, int32_t *num_dropped,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Rows a receive buffer needs for any routing of this shape and placement:
 * E * expert_capacity with a capacity, else T*k + min(E, T*k)*(alignment-1)
 * (each expert holding a pair pads by less than one alignment).  Pure host
 * arithmetic; -1 for invalid arguments.
 */
int64_t ep_layout_max_rows(int64_t num_tokens, int num_topk, int num_experts, int alignment,
                           int64_t expert_capacity);

/*
 * ep_dispatch -- permute (and optionally cast) token rows into the
 * expert-grouped receive buffer.
 *
 * Passages: NCCL EP page, nccl_ep.cc, ncclEpDispatch (x bf16 [T, hidden]
 * with 16-byte rows; fp8 output with hidden/128 fp32 scales per row) and
 * the dense-to-sparse weight step that returns recv_topk_weights; DeepEP
 * page, dispatch() (returns recv_x and recv_topk_weights; FP8 data comes
 * with its scale factors).
 *
 * In:  x             bf16 [num_tokens, hidden] row-major.
 *      slot          int32 [num_tokens * num_topk] from ep_layout.
 *      topk_weights  fp32 [num_tokens * num_topk] or NULL.
 * Out: recv_x        EP_OUT_BF16: bf16 [rows, hidden], row slot[t,j] =
 *                    x[t] bit for bit.
 *                    EP_OUT_FP8_E4M3: bytes [rows, hidden]; per token and
 *                    128-channel block b, amax = max |x|, scale =
 *                    amax / 448 (fp32, correctly rounded), code = OCP E4M3
 *                    of x / scale (fp32 quotient, correctly rounded) with
 *                    round-to-nearest-even and saturation to +-448; a block
 *                    with amax == 0 gets scale 0 and zero codes.  amax
 *                    ignores NaN; a NaN quotient (NaN x, or infinite x in
 *                    a block whose amax is infinite) gives 0x7F with the
 *                    sign of x.
 *      recv_scales   fp32 [rows, hidden/128]; required for FP8, else NULL.
 *      recv_weights  fp32 [rows] or NULL: recv_weights[slot[t,j]] =
 *                    topk_weights[t,j] (needs topk_weights).
 * Only rows named by slot are written; rows = num_tokens * num_topk is
 * always enough.  hidden must be a positive multiple of 8 (of 128 for FP8),
 * at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch(const void *x, int64_t num_tokens, int hidden, int num_topk,
                        const int32_t *slot, const float *topk_weights, int out_dtype, void *recv_x,
                        float *recv_scales, float *recv_weights, void *stream);

/*
 * ep_dispatch_ex -- ep_dispatch with the 8-bit cast variants.  ep_dispatch
 * is ep_dispatch_ex(scale_format = EP_SCALE_FP32).
 *
 * Passages: NCCL EP page, nccl_ep.cc: datatypes ncclFloat8e4m3 and
 * ncclFloat8e5m2 (ncclDataTypeToCudaDataType; ncclEpDispatch FP8
 * detection), and the low-latency dispatch kernel's round_scale and
 * use_ue8m0 arguments (ncclEpDispatch low-latency branch).
 *
 *   out_dtype     EP_OUT_BF16, EP_OUT_FP8_E4M3 (largest finite 448) or
 *                 EP_OUT_FP8_E5M2 (largest finite 57344).
 *   scale_format  EP_SCALE_FP32: scale = amax / max_finite, code =
 *                 RNE-saturating cast of the correctly rounded x / scale.
 *                 EP_SCALE_FP32_POW2 / EP_SCALE_UE8M0: scale = 2^e as
 *                 above, code = RNE-saturating cast of x * 2^-e (exact);
 *                 recv_scales is fp32 [rows, hidden/128] or, for UE8M0,
 *                 bytes [rows, hidden/128].  bf16 output takes
 *                 EP_SCALE_FP32 only.
 *   scale_ld      0: recv_scales row-major [rows, hidden/128].  > 0:
 *                 column-major [hidden/128, scale_ld] (block b of row r at
 *                 b*scale_ld + r: each block's scales contiguous over rows,
 *                 the layout a grouped GEMM reads per K block -- DeepEP
 *                 page, dispatch() use_tma_aligned_col_major_sf); scale_ld
 *                 must be a multiple of 16 bytes' worth of scales (4 fp32, 16
 *                 UE8M0) and at least the layout's rows; entries of rows
 *                 nothing maps to are not written.  fp8 output only.
 * amax ignores NaN.  amax == 0: codes 0 and scale 0 (fp32) or byte 0.  An
 * infinite amax: scale inf (fp32) or byte 0xFF, finite x encode to signed
 * zero; a NaN quotient gives 0x7F with the sign of x (both formats).
 * Other arguments and errors as ep_dispatch.
 */
ep_status_t ep_dispatch_ex(const void *x, int64_t num_tokens, int hidden, int num_topk,
                           const int32_t *slot, const float *topk_weights, int out_dtype,
                           int scale_format, void *recv_x, void *recv_scales, float *recv_weights,
                           int64_t scale_ld, void *stream);

/*
 * ep_dispatch_colmajor_scales -- the 8-bit cast of ep_dispatch_ex with
 * column-major scales, written in two passes through a caller workspace so
 * that each block's column is written in runs of consecutive rows: first the
 * codes of every slot and each token's scale row once (into the workspace),
 * then one lane per receive row copies its token's scales into the columns.
 * (ep_dispatch_ex with scale_ld > 0 writes the same bytes in one pass, one
 * row's scales at a time.)
 *
 * Passages: DeepEP page, dispatch() use_tma_aligned_col_major_sf (scale
 * factors stored column-major for the grouped GEMM); NCCL EP page,
 * ncclEpDispatch (per-128-channel scales of the cast).
 *
 * In:  x, slot, topk_weights, out_dtype (EP_OUT_FP8_E4M3 / _E5M2) and
 *      scale_format as ep_dispatch_ex.
 *      src        int32 [num_rows]: the source token of each receive row
 *                 (ep_layout's src); entries of rows nothing maps to may hold
 *                 anything: a row is filled only when one of its token's
 *                 slots is that row.
 *      num_rows   rows of the receive buffers (e.g. T*k, or
 *                 ep_layout_max_rows for ep_layout_ex layouts).
 *      workspace  >= ep_dispatch_colmajor_workspace_size(...) bytes,
 *                 256-byte aligned, contents clobbered.
 * Out: recv_x codes as ep_dispatch_ex; recv_scales [hidden/128, scale_ld]
 *      (fp32, or bytes for UE8M0): block b of row r at b*scale_ld + r, for
 *      the rows a slot maps to; other entries untouched.  scale_ld >= num_rows,
 *      a multiple of 16 bytes' worth of scales.
 * Rows of at most 1024 channels take ep_dispatch_ex's one-pass path.
 */
size_t ep_dispatch_colmajor_workspace_size(int64_t num_tokens, int hidden, int scale_format);
ep_status_t ep_dispatch_colmajor_scales(const void *x, int64_t num_tokens, int hidden, int num_topk,
                                        const int32_t *slot, const int32_t *src,
                                        const float *topk_weights, int out_dtype, int scale_format,
                                        void *recv_x, void *recv_scales, float *recv_weights,
                                        int64_t scale_ld, int64_t num_rows, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * ep_dispatch_prequantized -- dispatch of tokens that are already 8-bit
 * floats with per-128-channel fp32 scales: the code row and the scale row of
 * each token are copied, bit for bit, to every unmasked slot (any 8-bit
 * format passes through).
 *
 * Passages: NCCL EP page, ncclEpDispatch high-throughput branch (FP8 is
 * detected from the input datatype; FP8 tokens require a 2-D fp32 scales
 * input); DeepEP page, dispatch() (x may be a (data, scale_factors) tuple).
 *
 * In:  x_q       bytes [num_tokens, hidden], 16-byte aligned.
 *      x_scales  fp32 [num_tokens, hidden/128].
 *      slot, topk_weights as ep_dispatch.
 * Out: recv_q [rows, hidden], recv_scales fp32 [rows, hidden/128] (scale_ld
 *      0) or column-major [hidden/128, scale_ld] (as ep_dispatch_ex),
 *      recv_weights [rows] or NULL.
 * hidden must be a positive multiple of 128, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch_prequantized(const void *x_q, const float *x_scales, int64_t num_tokens,
                                     int hidden, int num_topk, const int32_t *slot,
                                     const float *topk_weights, void *recv_q, float *recv_scales,
                                     float *recv_weights, int64_t scale_ld, void *stream);

/*
 * ep_dispatch_prequantized_colmajor -- ep_dispatch_prequantized with
 * column-major scales written in two passes: the code rows per slot, then
 * one lane per receive row copies its token's scales from x_scales (which
 * already holds each token's scale row once) into the columns, so each
 * column is written in runs of consecutive rows.  No workspace.
 * (ep_dispatch_prequantized with scale_ld > 0 writes the same bytes in one
 * pass, one row's scales at a time.)
 *
 * Passages: DeepEP page, dispatch() (x may be a (data, scale factors) pair;
 * use_tma_aligned_col_major_sf: scale factors stored column-major); NCCL EP
 * page, ncclEpDispatch high-throughput branch (FP8 input with a 2-D fp32
 * scales tensor).
 *
 * In:  x_q, x_scales, slot, topk_weights as ep_dispatch_prequantized.
 *      src        int32 [num_rows]: the source token of each receive row
 *                 (ep_layout's src); entries of rows nothing maps to may hold
 *                 anything: a row is filled only when one of its token's
 *                 slots is that row.
 *      num_rows   rows of the receive buffers.
 * Out: recv_q [rows, hidden] as ep_dispatch_prequantized; recv_scales fp32
 *      [hidden/128, scale_ld]: block b of row r at b*scale_ld + r, for the
 *      rows a slot maps to, other entries untouched; scale_ld >= num_rows,
 *      a multiple of 4; recv_weights [rows] or NULL.
 * hidden must be a positive multiple of 128, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch_prequantized_colmajor(const void *x_q, const float *x_scales,
                                              int64_t num_tokens, int hidden, int num_topk,
                                              const int32_t *slot, const int32_t *src,
                                              const float *topk_weights, void *recv_q,
                                              float *recv_scales, float *recv_weights,
                                              int64_t scale_ld, int64_t num_rows, void *stream);

/*
 * ep_combine -- weighted reduction of expert outputs back to token order.
 *
 * Passages: NCCL EP page, nccl_ep.cc, ncclEpCombine (low-latency branch:
 * bf16 expert outputs reduced into [T, hidden] bf16 with topk_weights
 * [T, k] fp32; high-throughput forward combine: tokens only, no weights);
 * DeepEP page, combine().
 *
 * In:  y             bf16 [rows, hidden]: expert outputs, row r belongs to
 *                    the pair whose slot is r.
 *      slot          int32 [num_tokens * num_topk] from ep_layout.
 *      topk_weights  fp32 [num_tokens * num_topk] or NULL (all ones).
 * Out: out           bf16 [num_tokens, hidden]:
 *                    out[t] = bf16_rne( sum over j = 0..k-1 with slot >= 0
 *                    of w[t,j] * y[slot[t,j]] ), accumulated in fp32 with
 *                    one fused multiply-add per term in increasing j;
 *                    a token whose slots are all masked gets +0.
 * hidden must be a positive multiple of 8, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_combine(const void *y, const int32_t *slot, const float *topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, void *out, void *stream);

/*
 * ep_combine_backward -- gradients of ep_combine.
 *
 * Passages: DeepEP page, "MoE Dispatch and Combine for Training/Inference
 * with ElasticBuffer" (the backward of combine is a dispatch); NeMo
 * fused_a2a page, HybridEPCombine.backward (redispatch the combined-output
 * gradients through the saved layout); NCCL EP page, ncclEpCombine
 * high-throughput branch (backward combine with topk weight gradients).
 *
 * With out[t] = sum_j w[t,j] * y[slot[t,j]] and grad_out g:
 * In:  grad_out          bf16 [num_tokens, hidden].
 *      y                 bf16 [rows, hidden], the forward's expert outputs;
 *                        may be NULL when grad_topk_weights is NULL.
 *      slot              int32 [num_tokens * num_topk] from ep_layout.
 *      topk_weights      fp32 [num_tokens * num_topk] or NULL (all ones).
 * Out: grad_y            bf16 [rows, hidden]: grad_y[slot[t,j]] =
 *                        bf16_rne(w[t,j] * g[t]), one rounding of the exact
 *                        product (exact for products that are not fp32
 *                        subnormals); rows nothing maps to are not written.
 *      grad_topk_weights fp32 [num_tokens * num_topk] or NULL:
 *                        sum_c g[t,c] * y[slot[t,j],c] accumulated in fp32
 *                        (in an unspecified order), 0 for a masked pair.
 */
ep_status_t ep_combine_backward(const void *grad_out, const void *y, const int32_t *slot,
                                const float *topk_weights, int64_t num_tokens, int hidden,
                                int num_topk, void *grad_y, float *grad_topk_weights, void *stream);

/*
 * ep_dispatch_backward -- gradients of ep_dispatch.
 *
 * Passages: DeepEP page, "MoE Dispatch and Combine for Training/Inference
 * with ElasticBuffer" (the backward of dispatch is a combine that also
 * reduces the weight gradients); NeMo fused_a2a page,
 * HybridEPDispatch.backward.
 *
 * In:  grad_recv          bf16 [rows, hidden]: gradient of recv_x.
 *      grad_recv_weights  fp32 [rows] or NULL: gradient of recv_weights.
 *      slot               int32 [num_tokens * num_topk] from ep_layout.
 * Out: grad_x             bf16 [num_tokens, hidden]: bf16_rne of the fp32 sum
 *                         over unmasked j (ascending) of grad_recv[slot[t,j]]
 *                         -- ep_combine with unit weights.
 *      grad_topk_weights  fp32 [num_tokens * num_topk] or NULL (exactly when
 *                         grad_recv_weights is NULL): grad_recv_weights[slot],
 *                         0 for a masked pair.
 */
ep_status_t ep_dispatch_backward(const void *grad_recv, const float *grad_recv_weights,
                                 const int32_t *slot, int64_t num_tokens, int hidden, int num_topk,
                                 void *grad_x, float *grad_topk_weights, void *stream);

/*
 * ---- The per-(token, rank) path: a token travels once to each rank that
 * owns any of its experts.
 *
 * Passages: NCCL EP page, nccl_ep.cc: the high-throughput handle's routing
 * structures (the all-gathered routing bitmap, one bit per expert and eight
 * experts per byte; sparse_to_dense_map, the row of a (token, destination
 * rank) pair in that rank's buffer, -1 when not routed;
 * local_expert_routing_map, which local experts each received token
 * selects; num_tokens_for_experts, received tokens counted once per rank),
 * ncclEpCreateHandle's high-throughput branch (Step 1 bitmap, Step 2
 * all-gather, Step 3 metadata preprocessing with the per-expert receive
 * counter), and the high-throughput branches of ncclEpDispatch and
 * ncclEpCombine.
 *
 * Notation: G ranks (1..EP_MAX_RANKS, dividing E); rank d owns experts
 * [d*El, (d+1)*El), El = E / G.  Every rank contributes T rows to the
 * all-gathered map [G*T, W], W = ceil(E/8) bytes a row; global token
 * g = s*T + t is token t of rank s.  Rank d's receive buffer lists the
 * tokens that select any of its experts, once each, in increasing g.
 */

/*
 * ep_routing_map -- Step 1: the routing bitmap of one rank's tokens.
 * In:  topk_idx  int64 [num_tokens, num_topk], -1 = masked.
 * Out: routing_map  bytes [num_tokens, ceil(num_experts/8)]: bit e % 8 of
 *                   byte e / 8 of row t is 1 iff some slot of token t
 *                   selects expert e (duplicates select it once).
 *      num_invalid  int32 [1] or NULL: entries outside [-1, E).
 * Requires num_tokens * num_topk < 2^31, 1 <= num_topk <= EP_MAX_TOPK,
 * 1 <= num_experts <= EP_MAX_EXPERTS.
 */
ep_status_t ep_routing_map(const int64_t *topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, uint8_t *routing_map, int32_t *num_invalid,
                           void *stream);

/* Bytes of device workspace ep_rank_layout needs (int32 counts per chunk of
 * 1024 or more global tokens). */
size_t ep_rank_layout_workspace_size(int64_t tokens_per_rank, int num_experts, int num_ranks);

/*
 * ep_rank_layout -- Step 3 (metadata preprocessing) for rank `rank`.
 * In:  global_routing_map  bytes [G*T, W]: every rank's ep_routing_map rows,
 *                          rank s's at rows [s*T, (s+1)*T) (a rank with
 *                          fewer tokens pads with zero rows).
 *      k_out               width of recv_topk_idx, 1..EP_MAX_TOPK (num_topk
 *                          is always wide enough).
 * Out: sparse_to_dense_map  int32 [T, G]: row of this rank's token t in rank
 *                           d's buffer, -1 if t selects none of d's experts.
 *      num_recv             int32 [1]: tokens this rank receives.
 *      for received row i < num_recv (global token g):
 *        local_expert_routing_map  bytes [G*T, El]: 1 iff g selects local
 *                                  expert e (expert rank*El + e), else 0;
 *        recv_src                  int32 [G*T]: g;
 *        recv_topk_idx             int64 [G*T, k_out]: the selected local
 *                                  experts in increasing order, then -1;
 *      rows num_recv .. G*T-1: local map 0, recv_src -1, recv_topk_idx -1,
 *      so the three can be used at their full G*T rows (ep_layout over
 *      recv_topk_idx with E = El groups the received rows by local expert).
 *      expert_counts            int32 [El]: received tokens per local expert.
 *      num_overflow             int32 [1] or NULL: selections past k_out
 *                               (dropped from recv_topk_idx only).
 *      workspace                ep_rank_layout_workspace_size bytes, device.
 * Requires G*T < 2^31; local_expert_routing_map 4-byte aligned.
 */
ep_status_t ep_rank_layout(const uint8_t *global_routing_map, int64_t tokens_per_rank,
                           int num_experts, int num_ranks, int rank, int k_out,
                           int32_t *sparse_to_dense_map, uint8_t *local_expert_routing_map,
                           int32_t *recv_src, int64_t *recv_topk_idx, int32_t *expert_counts,
                           int32_t *num_recv, int32_t *num_overflow, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * ep_dispatch_ranked -- send this rank's tokens, once per destination rank.
 * In:  x                    bf16 [num_tokens, hidden].
 *      topk_idx, topk_weights  int64 / fp32 [num_tokens, num_topk]; read
 *                           only for dest_weights (topk_weights NULL = 1).
 *      sparse_to_dense_map  int32 [num_tokens, G] from ep_rank_layout.
 *      dest_x               HOST array of G device pointers: rank d's
 *                           receive buffer, bf16 [dest_rows, hidden] (on
 *                           one device, or peer memory mapped into it).
 *      dest_weights         NULL, or HOST array of G device pointers (an
 *                           entry may be NULL): fp32 [dest_rows, num_topk].
 * Out: dest_x[d][row] = x[t] for row = sparse_to_dense_map[t, d] >= 0;
 *      dest_weights[d][row, n] = the fp32 sum, in increasing slot order, of
 *      the weights of the slots selecting the n-th selected expert of rank d
 *      (increasing expert id, the order of recv_topk_idx), 0 past the last.
 *      Rows >= dest_rows are never written (G*T rows always suffice).
 * hidden must be a positive multiple of 8, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch_ranked(const void *x, const int64_t *topk_idx, const float *topk_weights,
                               int64_t num_tokens, int hidden, int num_topk, int num_experts,
                               int num_ranks, const int32_t *sparse_to_dense_map,
                               void *const *dest_x, float *const *dest_weights, int64_t dest_rows,
                               void *stream);

/*
 * ep_dispatch_ranked_prequantized -- ep_dispatch_ranked for tokens already
 * cast to 8 bits: each token's code row (hidden bytes) and scale row
 * (hidden/128 fp32) go to every destination rank that receives it, bit for
 * bit (any 8-bit format passes through).
 *
 * Passages: NCCL EP page, ncclEpDispatch high-throughput branch (FP8 tokens
 * need a 2-D fp32 scales tensor and travel as they are); DeepEP page,
 * dispatch() (x may be a (data, scale factors) pair).
 *
 * In:  x_q bytes [num_tokens, hidden] (16-byte aligned), x_scales fp32
 *      [num_tokens, hidden/128]; other inputs as ep_dispatch_ranked.
 * Out: dest_q      HOST array of G device pointers: bytes [dest_rows, hidden].
 *      dest_scales HOST array of G device pointers: fp32 [dest_rows, hidden/128].
 *      dest_weights as ep_dispatch_ranked.
 * hidden must be a positive multiple of 128, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch_ranked_prequantized(const void *x_q, const float *x_scales,
                                            const int64_t *topk_idx, const float *topk_weights,
                                            int64_t num_tokens, int hidden, int num_topk,
                                            int num_experts, int num_ranks,
                                            const int32_t *sparse_to_dense_map, void *const *dest_q,
                                            float *const *dest_scales, float *const *dest_weights,
                                            int64_t dest_rows, void *stream);

/*
 * ep_dispatch_ranked_fp8 -- ep_dispatch_ranked with the 8-bit cast of
 * ep_dispatch_ex done on the way: each token is cast once (per 128-channel
 * block: amax, scale, codes) and its code row and scale row go to every
 * destination rank that receives it.  The same bytes as ep_dispatch_ex of
 * the token followed by ep_dispatch_ranked_prequantized, without the
 * intermediate buffers.
 *
 * Passages: NCCL EP page, ncclEpDispatch: its low-latency branch casts
 * inside the dispatch (fp8 output with hidden/128 fp32 scales per token,
 * scale block 128; round_scale, use_ue8m0) and its high-throughput branch
 * sends a token once per rank; DeepEP page, ElasticBuffer
 * (use_fp8_dispatch).
 *
 * In:  x bf16 [num_tokens, hidden] (16-byte aligned); topk_idx,
 *      topk_weights, sparse_to_dense_map as ep_dispatch_ranked.
 *      out_dtype   EP_OUT_FP8_E4M3 or EP_OUT_FP8_E5M2.
 *      scale_format  as ep_dispatch_ex.
 * Out: dest_q      HOST array of G device pointers: codes [dest_rows, hidden]
 *                  (16-byte aligned).
 *      dest_scales HOST array of G device pointers: [dest_rows, hidden/128],
 *                  fp32 (4-byte aligned) or, for EP_SCALE_UE8M0, bytes.
 *      dest_weights as ep_dispatch_ranked (may be NULL).
 *      Row sparse_to_dense_map[t, d] (when >= 0 and < dest_rows) of rank d's
 *      buffers gets token t's codes and scales, exactly as ep_dispatch_ex
 *      casts them.
 * hidden must be a positive multiple of 128, at most EP_MAX_HIDDEN;
 * EP_UNSUPPORTED when the launch would need 2^31 workgroups or more (one per
 * token, tile of 64 or 128 units of 16 channels, and group of 8 ranks).
 */
ep_status_t ep_dispatch_ranked_fp8(const void *x, const int64_t *topk_idx, const float *topk_weights,
                                   int64_t num_tokens, int hidden, int num_topk, int num_experts,
                                   int num_ranks, const int32_t *sparse_to_dense_map,
                                   int out_dtype, int scale_format, void *const *dest_q,
                                   void *const *dest_scales, float *const *dest_weights,
                                   int64_t dest_rows, void *stream);

/*
 * ep_dispatch_fused_permute -- the receiving rank's dispatch with the
 * permute fused in: every token it receives is read once from the sending
 * rank's rows and written to each of its local-expert rows, so the rows come
 * out grouped by local expert with no intermediate receive buffer.
 *
 * Passages: NeMo fused_a2a page, HybridEPDispatch (fuse_permute; the
 * dispatched rows are grouped by local expert; pad_multiple); NCCL EP page,
 * sparse_to_dense_map / local_expert_routing_map.
 *
 * In:  src_x              HOST array of G device pointers: rank s's tokens,
 *                         bf16 [tokens_per_rank, hidden] (on one device, or
 *                         peer memory mapped into it).
 *      src_topk_idx       HOST array of G device pointers to rank s's int64
 *                         topk_idx [tokens_per_rank, num_topk]; read only for
 *                         recv_weights (may be NULL without them).
 *      src_topk_weights   NULL (unit weights), or HOST array of G device
 *                         pointers to fp32 [tokens_per_rank, num_topk]
 *                         (an entry may be NULL: unit weights).
 *      recv_src, recv_topk_idx  from ep_rank_layout for `rank` (k_out =
 *                         num_topk), all G*T rows.
 *      num_recv           NULL, or device int32 [1] (ep_rank_layout's
 *                         num_recv): only received rows i < num_recv
 *                         (clamped to [0, G*T]) are visited, and the count is
 *                         read on the device (no host round trip); rows past
 *                         it are not read;
 *                         NULL visits all G*T rows.
 *      slot               int32 [G*T, num_topk]: ep_layout (or ep_layout_ex
 *                         with an alignment) of recv_topk_idx over E/G
 *                         experts.
 * Out: recv_x [rows, hidden]: recv_x[slot[i, j]] = src_x[s][t] for received
 *      row i (recv_src[i] = s*T + t) and slot[i, j] >= 0;
 *      recv_weights [rows] or NULL: the fp32 sum, in increasing slot order,
 *      of rank s's weights of the slots that select expert
 *      rank*E/G + recv_topk_idx[i, j].
 *      Rows past `rows` are never written; rows nothing maps to are not.
 *      A received row whose recv_src is not in [0, G*T), or past num_recv,
 *      is skipped.
 * hidden must be a positive multiple of 8, at most EP_MAX_HIDDEN.  With
 * tokens_per_rank = 0 nothing is read or written and no pointer is checked.
 */
ep_status_t ep_dispatch_fused_permute(const void *const *src_x, const int64_t *const *src_topk_idx,
                                      const float *const *src_topk_weights, int64_t tokens_per_rank,
                                      int hidden, int num_topk, int num_experts, int num_ranks,
                                      int rank, const int32_t *recv_src,
                                      const int64_t *recv_topk_idx, const int32_t *num_recv,
                                      const int32_t *slot, int64_t rows, void *recv_x,
                                      float *recv_weights, void *stream);

/*
 * ep_dispatch_fused_permute_prequantized -- ep_dispatch_fused_permute for
 * tokens the senders already cast to 8 bits: each received token's code row
 * (hidden bytes) and its scale row (hidden/128 fp32) are read once and
 * written, bit for bit, to each of the token's local-expert rows.
 *
 * Passages: NeMo fused_a2a page, init_hybrid_ep_buffer (fp8_dispatch: FP8
 * communication in the dispatch phase) and HybridEPDispatch (fuse_permute);
 * NCCL EP page, ncclEpDispatch high-throughput branch (FP8 tokens travel
 * with a 2-D fp32 scales tensor).
 *
 * In:  src_q       HOST array of G device pointers: rank s's code rows,
 *                  bytes [tokens_per_rank, hidden] (16-byte aligned).
 *      src_scales  HOST array of G device pointers: rank s's scale rows,
 *                  fp32 [tokens_per_rank, hidden/128] (4-byte aligned).
 *      the rest as ep_dispatch_fused_permute.
 * Out: recv_q [rows, hidden] bytes (16-byte aligned) and recv_scales
 *      [rows, hidden/128] fp32 (4-byte aligned): row slot[i, j] >= 0 of both
 *      gets received row i's code and scale rows;
 *      recv_weights as ep_dispatch_fused_permute.
 *      Rows past `rows` are never written; rows nothing maps to are not.
 * hidden must be a positive multiple of 128, at most EP_MAX_HIDDEN.  With
 * tokens_per_rank = 0 nothing is read or written and no pointer is checked.
 */
ep_status_t ep_dispatch_fused_permute_prequantized(
    const void *const *src_q, const float *const *src_scales, const int64_t *const *src_topk_idx,
    const float *const *src_topk_weights, int64_t tokens_per_rank, int hidden, int num_topk,
    int num_experts, int num_ranks, int rank, const int32_t *recv_src,
    const int64_t *recv_topk_idx, const int32_t *num_recv, const int32_t *slot, int64_t rows,
    void *recv_q, float *recv_scales, float *recv_weights, void *stream);

/*
 * ep_combine_ranked -- gather this rank's tokens back from every rank.
 * In:  src_y                HOST array of G device pointers: rank d's
 *                           per-token outputs, bf16 [src_rows, hidden] (each
 *                           already reduced over d's experts, weighted).
 *      sparse_to_dense_map  int32 [num_tokens, G] from ep_rank_layout.
 * Out: out  bf16 [num_tokens, hidden]: bf16_rne of the fp32 sum, in
 *      increasing d, of src_y[d][sparse_to_dense_map[t, d]] over the ranks
 *      that hold the token (rows >= src_rows read as 0); +0 if none.
 * hidden must be a positive multiple of 8, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_combine_ranked(const void *const *src_y, int64_t src_rows,
                              const int32_t *sparse_to_dense_map, int64_t num_tokens, int hidden,
                              int num_ranks, void *out, void *stream);

/*
 * ep_dispatch_ranked_backward -- backward of ep_dispatch_ranked for this
 * rank's tokens: the row gradients come back as the combine over ranks and
 * the receivers' weight gradients come back to [num_tokens, num_topk].
 *
 * Passages: NCCL EP page, ncclEpCombine high-throughput branch (the backward
 * combine carries the tokens and the top-k weight gradients: each receiver's
 * weight gradients are made dense keyed by local_expert_routing_map, then
 * the sender brings them back to [T, k] through its rows of the routing
 * map); DeepEP page, "MoE Dispatch and Combine for Training/Inference with
 * ElasticBuffer" (the backward of dispatch is a combine that also reduces
 * the weight gradients).
 *
 * In:  grad_recv_x        NULL, or HOST array of G device pointers: rank d's
 *                         row gradients, bf16 [src_rows, hidden].
 *      grad_recv_weights  NULL, or HOST array of G device pointers (an entry
 *                         may be NULL: its gradients read as 0): fp32
 *                         [src_rows, num_topk], entry n of a row the gradient
 *                         of that row's weight for its n-th listed local
 *                         expert (recv_topk_idx order, as ep_dispatch_ranked
 *                         wrote dest_weights).
 *      topk_idx           int64 [num_tokens, num_topk] (this rank's).
 *      sparse_to_dense_map int32 [num_tokens, G] from ep_rank_layout.
 * Out: grad_x             bf16 [num_tokens, hidden] (with grad_recv_x): as
 *                         ep_combine_ranked of the row gradients.
 *      grad_topk_weights  fp32 [num_tokens, num_topk] (with
 *                         grad_recv_weights): for slot j with expert e of
 *                         rank d = e / (E/G), the entry of receiver d's row
 *                         sparse_to_dense_map[t, d] for e; every slot that
 *                         selected e (duplicates included) gets it.  0 for a
 *                         masked or invalid slot or a row outside
 *                         [0, src_rows).
 * At least one of the two pairs is given; hidden (with grad_recv_x) must be
 * a positive multiple of 8, at most EP_MAX_HIDDEN.
 */
ep_status_t ep_dispatch_ranked_backward(const void *const *grad_recv_x,
                                        const float *const *grad_recv_weights, int64_t src_rows,
                                        const int64_t *topk_idx, const int32_t *sparse_to_dense_map,
                                        int64_t num_tokens, int hidden, int num_topk,
                                        int num_experts, int num_ranks, void *grad_x,
                                        float *grad_topk_weights, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H_ */

// ep_internal.h -- launchers shared between the C ABI (ep_api.hip) and the
// kernel files.  Host-side declarations only; every launcher assumes the
// arguments were validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Layout: pairs are processed in chunks of flat indices, one workgroup of
// kLayoutThreads per chunk in both launches.  Inputs of up to
// kLayoutSmallChunks * kLayoutMinChunk pairs are cut into about
// kLayoutSmallChunks chunks of at least one 256-pair batch (more workgroups,
// shorter chains); larger ones into chunks of at least kLayoutMinChunk
// pairs, never more than kLayoutMaxChunks of them, so the per-workgroup
// histogram pass stays bounded for any input size.
constexpr int kLayoutThreads = 256;
constexpr int64_t kLayoutMinChunk = 1024;
constexpr int64_t kLayoutSmallChunks = 64;
constexpr int64_t kLayoutMaxChunks = 256;

// Inputs of at most kLayoutSmallMaxPairs pairs (and at most 256 experts)
// take a single launch instead of the two chunked ones.
constexpr int64_t kLayoutSmallMaxPairs = 16384;

int64_t layout_chunk_pairs(int64_t pairs);
int64_t layout_num_chunks(int64_t pairs);
size_t layout_workspace_bytes(int64_t pairs, int num_experts);

// The layout's fixed per-device scratch (the no-allocation entry point):
// its size (every accepted shape: kLayoutMaxChunks chunks of
// EP_MAX_EXPERTS counts plus a count per chunk), and its device address on
// the current device.
constexpr int kLayoutScratchExperts = 1024;   // EP_MAX_EXPERTS
constexpr size_t kLayoutScratchBytes =
    ((size_t)kLayoutMaxChunks * kLayoutScratchExperts + kLayoutMaxChunks) * sizeof(int32_t);
size_t layout_scratch_bytes();
hipError_t layout_scratch(void** ptr);

hipError_t launch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                         int num_experts, int alignment, int capacity, int32_t* counts,
                         int32_t* offsets, int32_t* slot, int32_t* src, int32_t* num_invalid,
                         int32_t* num_dropped, void* workspace, hipStream_t stream);

hipError_t launch_dispatch_bf16(const void* x, int64_t num_tokens, int hidden, int num_topk,
                                const int32_t* slot, const float* topk_weights, void* recv_x,
                                float* recv_weights, hipStream_t stream);

// format: 0 OCP E4M3, 1 OCP E5M2; scale_mode: 0 fp32 amax/max_finite,
// 1 power of two (fp32), 2 power of two as a UE8M0 byte.  scale_ld: 0 for
// row-major scales [rows, hidden/128], else column-major [hidden/128,
// scale_ld].
hipError_t launch_dispatch_fp8(const void* x, int64_t num_tokens, int hidden, int num_topk,
                               const int32_t* slot, const float* topk_weights, int format,
                               int scale_mode, void* recv_q, void* recv_scales,
                               float* recv_weights, int64_t scale_ld, hipStream_t stream);

// The 8-bit cast with column-major scales in two passes: codes per slot
// and each token's scale row once into `workspace` (colmajor_workspace_bytes),
// then the scales written to [hidden/128, scale_ld] one receive row per lane
// (src: the source token of each of the `rows` receive rows).
size_t colmajor_workspace_bytes(int64_t num_tokens, int hidden, int scale_mode);
hipError_t launch_dispatch_fp8_colmajor(const void* x, int64_t num_tokens, int hidden,
                                        int num_topk, const int32_t* slot, const int32_t* src,
                                        const float* topk_weights, int format, int scale_mode,
                                        void* recv_q, void* recv_scales, float* recv_weights,
                                        int64_t scale_ld, int64_t rows, void* workspace,
                                        hipStream_t stream);

hipError_t launch_dispatch_prequant(const void* xq, const float* xs, int64_t num_tokens,
                                    int hidden, int num_topk, const int32_t* slot,
                                    const float* topk_weights, void* recv_q, float* recv_scales,
                                    float* recv_weights, int64_t scale_ld, hipStream_t stream);

// Pre-quantized rows with column-major scales in two passes: the code rows
// per slot, then the scales of each of the `rows` receive rows from its
// token's row of xs (src: the source token of each receive row).
hipError_t launch_dispatch_prequant_colmajor(const void* xq, const float* xs, int64_t num_tokens,
                                             int hidden, int num_topk, const int32_t* slot,
                                             const int32_t* src, const float* topk_weights,
                                             void* recv_q, float* recv_scales, float* recv_weights,
                                             int64_t scale_ld, int64_t rows, hipStream_t stream);

// row_w / out_w: optional gather out_w[t,j] = row_w[slot[t,j]] (dispatch
// backward); both NULL for a plain combine.
hipError_t launch_combine(const void* y, const int32_t* slot, const float* topk_weights,
                          int64_t num_tokens, int hidden, int num_topk, void* out,
                          const float* row_w, float* out_w, hipStream_t stream);

// ---- per-(token, rank) path (ep_ranked.hip)

constexpr int kMaxRanks = 64;  // EP_MAX_RANKS

// G device row pointers, passed by value as a kernel argument (a rank's
// buffer may be NULL where the call allows it).
struct RankPtrs {
    void* p[kMaxRanks];
};

hipError_t launch_routing_map(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                              int num_experts, uint8_t* map, int32_t* num_invalid,
                              hipStream_t stream);

size_t rank_layout_workspace_bytes(int64_t tokens_per_rank, int num_experts, int num_ranks);

hipError_t launch_rank_layout(const uint8_t* map, int64_t tokens_per_rank, int num_experts,
                              int num_ranks, int rank, int k_out, int32_t* s2d,
                              uint8_t* local_map, int32_t* recv_src, int64_t* recv_topk_idx,
                              int32_t* expert_counts, int32_t* num_recv, int32_t* num_overflow,
                              void* workspace, hipStream_t stream);

// Rows of row_bytes (a multiple of 16): bf16 tokens or 8-bit codes; with
// x_scales, num_scales fp32 per token are copied to dest_scales too.
hipError_t launch_dispatch_ranked(const void* x, const int64_t* topk_idx, const float* topk_weights,
                                  int64_t num_tokens, int row_bytes, int num_topk, int num_experts,
                                  int num_ranks, const int32_t* s2d, const RankPtrs& dest_x,
                                  const RankPtrs& dest_w, bool with_weights, const float* x_scales,
                                  const RankPtrs& dest_scales, int num_scales, int64_t dest_rows,
                                  hipStream_t stream);

// The 8-bit cast of ep_dispatch_ex sent once per destination rank: codes
// [dest_rows, hidden] and scale rows [dest_rows, hidden/128] (fp32, or UE8M0
// bytes) per rank.  ranked_fp8_blocks: the workgroups it launches (the call
// fails past INT32_MAX).
int64_t ranked_fp8_blocks(int64_t num_tokens, int hidden, int num_ranks);
hipError_t launch_dispatch_ranked_fp8(const void* x, const int64_t* topk_idx,
                                      const float* topk_weights, int64_t num_tokens, int hidden,
                                      int num_topk, int num_experts, int num_ranks,
                                      const int32_t* s2d, int format, int scale_mode,
                                      const RankPtrs& dest_q, const RankPtrs& dest_scales,
                                      const RankPtrs& dest_w, bool with_weights, int64_t dest_rows,
                                      hipStream_t stream);

hipError_t launch_dispatch_fused_permute(const RankPtrs& src_x, const RankPtrs& src_idx,
                                         const RankPtrs& src_w, int64_t tokens_per_rank,
                                         int hidden, int num_topk, int num_experts, int num_ranks,
                                         int rank, const int32_t* recv_src,
                                         const int64_t* recv_topk_idx, const int32_t* num_recv,
                                         const int32_t* slot, int64_t rows, void* recv_x,
                                         float* recv_w, hipStream_t stream);

// The same for 8-bit code rows (hidden bytes) with their fp32 scale rows
// (hidden / 128 per token, row-major on both sides).
hipError_t launch_dispatch_fused_permute_prequant(const RankPtrs& src_q, const RankPtrs& src_s,
                                                  const RankPtrs& src_idx, const RankPtrs& src_w,
                                                  int64_t tokens_per_rank, int hidden,
                                                  int num_topk, int num_experts, int num_ranks,
                                                  int rank, const int32_t* recv_src,
                                                  const int64_t* recv_topk_idx,
                                                  const int32_t* num_recv, const int32_t* slot,
                                                  int64_t rows, void* recv_q, float* recv_s,
                                                  float* recv_w, hipStream_t stream);

hipError_t launch_combine_ranked(const RankPtrs& src_y, int64_t src_rows, const int32_t* s2d,
                                 int64_t num_tokens, int hidden, int num_ranks, void* out,
                                 hipStream_t stream);

// grad_topk_weights[t, j] from the receivers' [src_rows, num_topk] weight
// gradients (backward of the once-per-rank dispatch).
hipError_t launch_ranked_weight_grad(const RankPtrs& grad_w, int64_t src_rows,
                                     const int64_t* topk_idx, const int32_t* s2d,
                                     int64_t num_tokens, int num_topk, int num_experts,
                                     int num_ranks, float* grad_topk_weights, hipStream_t stream);

hipError_t launch_combine_backward(const void* grad_out, const void* y, const int32_t* slot,
                                   const float* topk_weights, int64_t num_tokens, int hidden,
                                   int num_topk, void* grad_y, float* grad_topk_weights,
                                   hipStream_t stream);

}  // namespace ep

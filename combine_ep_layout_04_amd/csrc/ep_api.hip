// ep_api.hip -- the C ABI declared in include/ep.h: argument checks on the
// host, then stream-ordered launches.  Nothing here allocates, frees or
// synchronises; every failure is a returned status code (the pages' host
// library maps CUDA errors to an internal-error code and returns invalid-
// argument / invalid-usage codes; it never has to exit for bad input here).

#include <stdarg.h>
#include <stdio.h>

#include "ep.h"
#include "ep_internal.h"

static_assert(EP_LAYOUT_NOALLOC_SCRATCH_BYTES == ep::kLayoutScratchBytes,
              "the header states the layout scratch size");
static_assert(EP_MAX_EXPERTS == ep::kLayoutScratchExperts, "the scratch covers every expert count");

namespace {

thread_local char g_last_error[256] = "";

ep_status_t fail(ep_status_t status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

ep_status_t from_hip(hipError_t err, const char* what)
{
    if (err == hipSuccess) return EP_SUCCESS;
    return fail(EP_RUNTIME_ERROR, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ep_status_t check_tokens(int64_t num_tokens, int num_topk)
{
    if (num_tokens < 0) return fail(EP_INVALID_ARGUMENT, "num_tokens < 0");
    if (num_topk < 1 || num_topk > EP_MAX_TOPK)
        return fail(EP_INVALID_ARGUMENT, "num_topk %d outside [1, %d]", num_topk, EP_MAX_TOPK);
    if (num_tokens * (int64_t)num_topk >= ((int64_t)1 << 31))
        return fail(EP_UNSUPPORTED, "num_tokens * num_topk must be < 2^31");
    return EP_SUCCESS;
}

ep_status_t check_hidden(int hidden, int multiple)
{
    if (hidden < 1 || hidden > EP_MAX_HIDDEN || hidden % multiple != 0)
        return fail(EP_INVALID_ARGUMENT, "hidden %d must be a positive multiple of %d, at most %d",
                    hidden, multiple, EP_MAX_HIDDEN);
    return EP_SUCCESS;
}

}  // namespace

extern "C" {

int ep_version(void) { return (1 << 16) | 0; }

const char* ep_status_string(int status)
{
    switch (status) {
    case EP_SUCCESS: return "EP_SUCCESS";
    case EP_INVALID_ARGUMENT: return "EP_INVALID_ARGUMENT";
    case EP_UNSUPPORTED: return "EP_UNSUPPORTED";
    case EP_RUNTIME_ERROR: return "EP_RUNTIME_ERROR";
    default: return "EP_UNKNOWN_STATUS";
    }
}

const char* ep_last_error(void) { return g_last_error; }

size_t ep_layout_workspace_size(int64_t num_tokens, int num_topk, int num_experts)
{
    if (num_tokens < 0 || num_topk < 1 || num_topk > EP_MAX_TOPK || num_experts < 1 ||
        num_experts > EP_MAX_EXPERTS || num_tokens * (int64_t)num_topk >= ((int64_t)1 << 31))
        return 0;
    return ep::layout_workspace_bytes(num_tokens * (int64_t)num_topk, num_experts);
}

int64_t ep_layout_max_rows(int64_t num_tokens, int num_topk, int num_experts, int alignment,
                           int64_t expert_capacity)
{
    if (num_tokens < 0 || num_topk < 1 || num_topk > EP_MAX_TOPK || num_experts < 1 ||
        num_experts > EP_MAX_EXPERTS || alignment < 1 || alignment > EP_MAX_ALIGNMENT ||
        expert_capacity < 0 || (expert_capacity > 0 && expert_capacity % alignment != 0) ||
        num_tokens * (int64_t)num_topk >= ((int64_t)1 << 31))
        return -1;
    const int64_t pairs = num_tokens * (int64_t)num_topk;
    if (expert_capacity > 0) return (int64_t)num_experts * expert_capacity;
    // every expert with at least one pair may add up to alignment-1 rows
    const int64_t touched = pairs < num_experts ? pairs : num_experts;
    return pairs + touched * (alignment - 1);
}

ep_status_t ep_layout_ex(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                         int alignment, int64_t expert_capacity, int32_t* counts, int32_t* offsets,
                         int32_t* slot, int32_t* src, int32_t* num_invalid, int32_t* num_dropped,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
        return fail(EP_INVALID_ARGUMENT, "num_experts %d outside [1, %d]", num_experts,
                    EP_MAX_EXPERTS);
    if (alignment < 1 || alignment > EP_MAX_ALIGNMENT)
        return fail(EP_INVALID_ARGUMENT, "alignment %d outside [1, %d]", alignment,
                    EP_MAX_ALIGNMENT);
    if (expert_capacity < 0 || (expert_capacity > 0 && expert_capacity % alignment != 0))
        return fail(EP_INVALID_ARGUMENT,
                    "expert_capacity %lld must be 0 or a positive multiple of alignment %d",
                    (long long)expert_capacity, alignment);
    const int64_t rows = ep_layout_max_rows(num_tokens, num_topk, num_experts, alignment,
                                            expert_capacity);
    if (rows < 0 || rows >= ((int64_t)1 << 31))
        return fail(EP_UNSUPPORTED, "the layout could need %lld rows; rows must stay below 2^31",
                    (long long)rows);
    if (!counts || !offsets) return fail(EP_INVALID_ARGUMENT, "counts and offsets are required");
    if (num_tokens > 0 && (!topk_idx || !slot))
        return fail(EP_INVALID_ARGUMENT, "topk_idx and slot are required");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(EP_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    const size_t need = ep_layout_workspace_size(num_tokens, num_topk, num_experts);
    if (workspace_bytes < need)
        return fail(EP_INVALID_ARGUMENT, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(topk_idx) & 7u))
        return fail(EP_INVALID_ARGUMENT, "topk_idx must be 8-byte aligned");
    return from_hip(ep::launch_layout(topk_idx, num_tokens, num_topk, num_experts, alignment,
                                      (int)expert_capacity, counts, offsets, slot, src,
                                      num_invalid, num_dropped, workspace,
                                      static_cast<hipStream_t>(stream)),
                    "ep_layout launch");
}

ep_status_t ep_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                      int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src,
                      int32_t* num_invalid, void* workspace, size_t workspace_bytes, void* stream)
{
    return ep_layout_ex(topk_idx, num_tokens, num_topk, num_experts, 1, 0, counts, offsets, slot,
                        src, num_invalid, nullptr, workspace, workspace_bytes, stream);
}

ep_status_t ep_layout_noalloc(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                              int num_experts, int32_t* counts, int32_t* offsets, int32_t* slot,
                              int32_t* src, int32_t* num_invalid, void* stream)
{
    g_last_error[0] = '\0';
    const size_t need = ep_layout_workspace_size(num_tokens, num_topk, num_experts);
    if (need == 0)   // an invalid shape: ep_layout_ex names the argument, before any HIP call
        return ep_layout_ex(topk_idx, num_tokens, num_topk, num_experts, 1, 0, counts, offsets,
                            slot, src, num_invalid, nullptr, nullptr, 0, stream);
    const size_t have = ep::layout_scratch_bytes();
    if (need > have)
        return fail(EP_UNSUPPORTED,
                    "ep_layout_noalloc: this shape needs %zu bytes of scratch, more than the %zu "
                    "bytes the library holds per device",
                    need, have);
    void* scratch = nullptr;
    const ep_status_t st = from_hip(ep::layout_scratch(&scratch), "ep_layout_noalloc scratch address");
    if (st) return st;
    return ep_layout_ex(topk_idx, num_tokens, num_topk, num_experts, 1, 0, counts, offsets, slot,
                        src, num_invalid, nullptr, scratch, have, stream);
}

// scale_ld: 0, or a positive multiple of the 16-byte column alignment
static ep_status_t check_scale_ld(int64_t scale_ld, int elem_bytes)
{
    const int64_t align = 16 / elem_bytes;
    if (scale_ld < 0 || (scale_ld > 0 && scale_ld % align != 0))
        return fail(EP_INVALID_ARGUMENT,
                    "scale_ld %lld must be 0 (row-major) or a positive multiple of %lld",
                    (long long)scale_ld, (long long)align);
    return EP_SUCCESS;
}

ep_status_t ep_dispatch_ex(const void* x, int64_t num_tokens, int hidden, int num_topk,
                           const int32_t* slot, const float* topk_weights, int out_dtype,
                           int scale_format, void* recv_x, void* recv_scales, float* recv_weights,
                           int64_t scale_ld, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    if (out_dtype != EP_OUT_BF16 && out_dtype != EP_OUT_FP8_E4M3 && out_dtype != EP_OUT_FP8_E5M2)
        return fail(EP_INVALID_ARGUMENT, "unknown out_dtype %d", out_dtype);
    if (scale_format != EP_SCALE_FP32 && scale_format != EP_SCALE_FP32_POW2 &&
        scale_format != EP_SCALE_UE8M0)
        return fail(EP_INVALID_ARGUMENT, "unknown scale_format %d", scale_format);
    const bool fp8 = out_dtype != EP_OUT_BF16;
    if (!fp8 && scale_format != EP_SCALE_FP32)
        return fail(EP_INVALID_ARGUMENT, "bf16 output takes no scale format");
    st = check_hidden(hidden, fp8 ? 128 : 8);
    if (st) return st;
    if (!fp8 && scale_ld != 0) return fail(EP_INVALID_ARGUMENT, "bf16 output takes no scale_ld");
    st = check_scale_ld(scale_ld, scale_format == EP_SCALE_UE8M0 ? 1 : 4);
    if (st) return st;
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x || !slot || !recv_x) return fail(EP_INVALID_ARGUMENT, "x, slot and recv_x are required");
    if (!aligned16(x) || !aligned16(recv_x))
        return fail(EP_INVALID_ARGUMENT, "x and recv_x must be 16-byte aligned");
    if (recv_weights && !topk_weights)
        return fail(EP_INVALID_ARGUMENT, "recv_weights needs topk_weights");
    if (fp8) {
        if (!recv_scales) return fail(EP_INVALID_ARGUMENT, "fp8 dispatch needs recv_scales");
        if (scale_format != EP_SCALE_UE8M0 && (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
            return fail(EP_INVALID_ARGUMENT, "fp32 recv_scales must be 4-byte aligned");
        return from_hip(ep::launch_dispatch_fp8(x, num_tokens, hidden, num_topk, slot, topk_weights,
                                                out_dtype == EP_OUT_FP8_E5M2 ? 1 : 0, scale_format,
                                                recv_x, recv_scales, recv_weights, scale_ld,
                                                static_cast<hipStream_t>(stream)),
                        "ep_dispatch (fp8) launch");
    }
    if (recv_scales) return fail(EP_INVALID_ARGUMENT, "recv_scales must be NULL for bf16 output");
    return from_hip(ep::launch_dispatch_bf16(x, num_tokens, hidden, num_topk, slot, topk_weights,
                                             recv_x, recv_weights, static_cast<hipStream_t>(stream)),
                    "ep_dispatch (bf16) launch");
}

size_t ep_dispatch_colmajor_workspace_size(int64_t num_tokens, int hidden, int scale_format)
{
    if (num_tokens < 0 || hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0 ||
        (scale_format != EP_SCALE_FP32 && scale_format != EP_SCALE_FP32_POW2 &&
         scale_format != EP_SCALE_UE8M0))
        return 0;
    return ep::colmajor_workspace_bytes(num_tokens, hidden, scale_format);
}

ep_status_t ep_dispatch_colmajor_scales(const void* x, int64_t num_tokens, int hidden, int num_topk,
                                        const int32_t* slot, const int32_t* src,
                                        const float* topk_weights, int out_dtype, int scale_format,
                                        void* recv_x, void* recv_scales, float* recv_weights,
                                        int64_t scale_ld, int64_t num_rows, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    if (out_dtype != EP_OUT_FP8_E4M3 && out_dtype != EP_OUT_FP8_E5M2)
        return fail(EP_INVALID_ARGUMENT, "out_dtype %d: column-major scales come with an 8-bit cast",
                    out_dtype);
    if (scale_format != EP_SCALE_FP32 && scale_format != EP_SCALE_FP32_POW2 &&
        scale_format != EP_SCALE_UE8M0)
        return fail(EP_INVALID_ARGUMENT, "unknown scale_format %d", scale_format);
    st = check_hidden(hidden, 128);
    if (st) return st;
    if (scale_ld <= 0) return fail(EP_INVALID_ARGUMENT, "scale_ld must be positive (column-major)");
    st = check_scale_ld(scale_ld, scale_format == EP_SCALE_UE8M0 ? 1 : 4);
    if (st) return st;
    if (num_rows < 0 || num_rows > INT32_MAX)
        return fail(EP_INVALID_ARGUMENT, "num_rows %lld outside [0, 2^31-1] (slot entries are int32)",
                    (long long)num_rows);
    if (scale_ld < num_rows)
        return fail(EP_INVALID_ARGUMENT, "scale_ld %lld is below num_rows %lld", (long long)scale_ld,
                    (long long)num_rows);
    const size_t need = ep_dispatch_colmajor_workspace_size(num_tokens, hidden, scale_format);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(EP_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < need)
        return fail(EP_INVALID_ARGUMENT, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x || !slot || !src || !recv_x || !recv_scales)
        return fail(EP_INVALID_ARGUMENT, "x, slot, src, recv_x and recv_scales are required");
    if (!aligned16(x) || !aligned16(recv_x))
        return fail(EP_INVALID_ARGUMENT, "x and recv_x must be 16-byte aligned");
    if (scale_format != EP_SCALE_UE8M0 && (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
        return fail(EP_INVALID_ARGUMENT, "fp32 recv_scales must be 4-byte aligned");
    if (recv_weights && !topk_weights)
        return fail(EP_INVALID_ARGUMENT, "recv_weights needs topk_weights");
    return from_hip(ep::launch_dispatch_fp8_colmajor(
                        x, num_tokens, hidden, num_topk, slot, src, topk_weights,
                        out_dtype == EP_OUT_FP8_E5M2 ? 1 : 0, scale_format, recv_x, recv_scales,
                        recv_weights, scale_ld, num_rows, workspace,
                        static_cast<hipStream_t>(stream)),
                    "ep_dispatch_colmajor_scales launch");
}

ep_status_t ep_dispatch(const void* x, int64_t num_tokens, int hidden, int num_topk,
                        const int32_t* slot, const float* topk_weights, int out_dtype, void* recv_x,
                        float* recv_scales, float* recv_weights, void* stream)
{
    return ep_dispatch_ex(x, num_tokens, hidden, num_topk, slot, topk_weights, out_dtype,
                          EP_SCALE_FP32, recv_x, recv_scales, recv_weights, 0, stream);
}

ep_status_t ep_dispatch_prequantized(const void* x_q, const float* x_scales, int64_t num_tokens,
                                     int hidden, int num_topk, const int32_t* slot,
                                     const float* topk_weights, void* recv_q, float* recv_scales,
                                     float* recv_weights, int64_t scale_ld, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 128);
    if (st) return st;
    st = check_scale_ld(scale_ld, 4);
    if (st) return st;
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x_q || !x_scales || !slot || !recv_q || !recv_scales)
        return fail(EP_INVALID_ARGUMENT, "x_q, x_scales, slot, recv_q and recv_scales are required");
    if (!aligned16(x_q) || !aligned16(recv_q))
        return fail(EP_INVALID_ARGUMENT, "x_q and recv_q must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(x_scales) & 3u) || (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
        return fail(EP_INVALID_ARGUMENT, "scales must be 4-byte aligned");
    if (recv_weights && !topk_weights)
        return fail(EP_INVALID_ARGUMENT, "recv_weights needs topk_weights");
    return from_hip(ep::launch_dispatch_prequant(x_q, x_scales, num_tokens, hidden, num_topk, slot,
                                                 topk_weights, recv_q, recv_scales, recv_weights,
                                                 scale_ld, static_cast<hipStream_t>(stream)),
                    "ep_dispatch_prequantized launch");
}

ep_status_t ep_dispatch_prequantized_colmajor(const void* x_q, const float* x_scales,
                                              int64_t num_tokens, int hidden, int num_topk,
                                              const int32_t* slot, const int32_t* src,
                                              const float* topk_weights, void* recv_q,
                                              float* recv_scales, float* recv_weights,
                                              int64_t scale_ld, int64_t num_rows, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 128);
    if (st) return st;
    if (scale_ld <= 0) return fail(EP_INVALID_ARGUMENT, "scale_ld must be positive (column-major)");
    st = check_scale_ld(scale_ld, 4);
    if (st) return st;
    if (num_rows < 0 || num_rows > INT32_MAX)
        return fail(EP_INVALID_ARGUMENT, "num_rows %lld outside [0, 2^31-1] (slot entries are int32)",
                    (long long)num_rows);
    if (scale_ld < num_rows)
        return fail(EP_INVALID_ARGUMENT, "scale_ld %lld is below num_rows %lld", (long long)scale_ld,
                    (long long)num_rows);
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x_q || !x_scales || !slot || !src || !recv_q || !recv_scales)
        return fail(EP_INVALID_ARGUMENT,
                    "x_q, x_scales, slot, src, recv_q and recv_scales are required");
    if (!aligned16(x_q) || !aligned16(recv_q))
        return fail(EP_INVALID_ARGUMENT, "x_q and recv_q must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(x_scales) & 3u) || (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
        return fail(EP_INVALID_ARGUMENT, "scales must be 4-byte aligned");
    if (recv_weights && !topk_weights)
        return fail(EP_INVALID_ARGUMENT, "recv_weights needs topk_weights");
    return from_hip(ep::launch_dispatch_prequant_colmajor(
                        x_q, x_scales, num_tokens, hidden, num_topk, slot, src, topk_weights, recv_q,
                        recv_scales, recv_weights, scale_ld, num_rows,
                        static_cast<hipStream_t>(stream)),
                    "ep_dispatch_prequantized_colmajor launch");
}

ep_status_t ep_combine(const void* y, const int32_t* slot, const float* topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, void* out, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 8);
    if (st) return st;
    if (num_tokens == 0) return EP_SUCCESS;
    if (!y || !slot || !out) return fail(EP_INVALID_ARGUMENT, "y, slot and out are required");
    if (!aligned16(y) || !aligned16(out))
        return fail(EP_INVALID_ARGUMENT, "y and out must be 16-byte aligned");
    return from_hip(ep::launch_combine(y, slot, topk_weights, num_tokens, hidden, num_topk, out,
                                       nullptr, nullptr, static_cast<hipStream_t>(stream)),
                    "ep_combine launch");
}

ep_status_t ep_combine_backward(const void* grad_out, const void* y, const int32_t* slot,
                                const float* topk_weights, int64_t num_tokens, int hidden,
                                int num_topk, void* grad_y, float* grad_topk_weights, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 8);
    if (st) return st;
    if (num_tokens == 0) return EP_SUCCESS;
    if (!grad_out || !slot || !grad_y)
        return fail(EP_INVALID_ARGUMENT, "grad_out, slot and grad_y are required");
    if (grad_topk_weights && !y)
        return fail(EP_INVALID_ARGUMENT, "grad_topk_weights needs the expert outputs y");
    if (!aligned16(grad_out) || !aligned16(grad_y) || (y && !aligned16(y)))
        return fail(EP_INVALID_ARGUMENT, "grad_out, y and grad_y must be 16-byte aligned");
    return from_hip(ep::launch_combine_backward(grad_out, y, slot, topk_weights, num_tokens, hidden,
                                                num_topk, grad_y, grad_topk_weights,
                                                static_cast<hipStream_t>(stream)),
                    "ep_combine_backward launch");
}

ep_status_t ep_dispatch_backward(const void* grad_recv, const float* grad_recv_weights,
                                 const int32_t* slot, int64_t num_tokens, int hidden, int num_topk,
                                 void* grad_x, float* grad_topk_weights, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 8);
    if (st) return st;
    if (num_tokens == 0) return EP_SUCCESS;
    if (!grad_recv || !slot || !grad_x)
        return fail(EP_INVALID_ARGUMENT, "grad_recv, slot and grad_x are required");
    if ((grad_topk_weights == nullptr) != (grad_recv_weights == nullptr))
        return fail(EP_INVALID_ARGUMENT,
                    "grad_recv_weights and grad_topk_weights are given together or not at all");
    if (!aligned16(grad_recv) || !aligned16(grad_x))
        return fail(EP_INVALID_ARGUMENT, "grad_recv and grad_x must be 16-byte aligned");
    return from_hip(ep::launch_combine(grad_recv, slot, nullptr, num_tokens, hidden, num_topk,
                                       grad_x, grad_recv_weights, grad_topk_weights,
                                       static_cast<hipStream_t>(stream)),
                    "ep_dispatch_backward launch");
}


// ---- per-(token, rank) path

static ep_status_t check_ranks(int num_experts, int num_ranks)
{
    if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
        return fail(EP_INVALID_ARGUMENT, "num_experts %d outside [1, %d]", num_experts,
                    EP_MAX_EXPERTS);
    if (num_ranks < 1 || num_ranks > EP_MAX_RANKS)
        return fail(EP_INVALID_ARGUMENT, "num_ranks %d outside [1, %d]", num_ranks, EP_MAX_RANKS);
    if (num_experts % num_ranks != 0)
        return fail(EP_INVALID_ARGUMENT, "num_experts %d is not a multiple of num_ranks %d",
                    num_experts, num_ranks);
    return EP_SUCCESS;
}

ep_status_t ep_routing_map(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, uint8_t* routing_map, int32_t* num_invalid,
                           void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
        return fail(EP_INVALID_ARGUMENT, "num_experts %d outside [1, %d]", num_experts,
                    EP_MAX_EXPERTS);
    if (num_tokens > 0 && (!topk_idx || !routing_map))
        return fail(EP_INVALID_ARGUMENT, "topk_idx and routing_map are required");
    if ((reinterpret_cast<uintptr_t>(topk_idx) & 7u))
        return fail(EP_INVALID_ARGUMENT, "topk_idx must be 8-byte aligned");
    if ((reinterpret_cast<uintptr_t>(num_invalid) & 3u))
        return fail(EP_INVALID_ARGUMENT, "num_invalid must be 4-byte aligned");
    return from_hip(ep::launch_routing_map(topk_idx, num_tokens, num_topk, num_experts,
                                           routing_map, num_invalid,
                                           static_cast<hipStream_t>(stream)),
                    "ep_routing_map launch");
}

size_t ep_rank_layout_workspace_size(int64_t tokens_per_rank, int num_experts, int num_ranks)
{
    if (tokens_per_rank < 0 || num_ranks < 1 || num_ranks > EP_MAX_RANKS || num_experts < 1 ||
        num_experts > EP_MAX_EXPERTS || num_experts % num_ranks != 0)
        return 0;
    const size_t bytes = ep::rank_layout_workspace_bytes(tokens_per_rank, num_experts, num_ranks);
    return (bytes + 255) & ~(size_t)255;
}

ep_status_t ep_rank_layout(const uint8_t* global_routing_map, int64_t tokens_per_rank,
                           int num_experts, int num_ranks, int rank, int k_out,
                           int32_t* sparse_to_dense_map, uint8_t* local_expert_routing_map,
                           int32_t* recv_src, int64_t* recv_topk_idx, int32_t* expert_counts,
                           int32_t* num_recv, int32_t* num_overflow, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    if (tokens_per_rank < 0) return fail(EP_INVALID_ARGUMENT, "tokens_per_rank < 0");
    if (rank < 0 || rank >= num_ranks)
        return fail(EP_INVALID_ARGUMENT, "rank %d outside [0, %d)", rank, num_ranks);
    if (k_out < 1 || k_out > EP_MAX_TOPK)
        return fail(EP_INVALID_ARGUMENT, "k_out %d outside [1, %d]", k_out, EP_MAX_TOPK);
    if (tokens_per_rank * (int64_t)num_ranks >= ((int64_t)1 << 31))
        return fail(EP_UNSUPPORTED, "num_ranks * tokens_per_rank must be < 2^31");
    if (!expert_counts || !num_recv)
        return fail(EP_INVALID_ARGUMENT, "expert_counts and num_recv are required");
    if (tokens_per_rank > 0 && (!global_routing_map || !sparse_to_dense_map ||
                                !local_expert_routing_map || !recv_src || !recv_topk_idx))
        return fail(EP_INVALID_ARGUMENT,
                    "global_routing_map, sparse_to_dense_map, local_expert_routing_map, recv_src "
                    "and recv_topk_idx are required");
    if ((reinterpret_cast<uintptr_t>(local_expert_routing_map) & 3u) ||
        (reinterpret_cast<uintptr_t>(sparse_to_dense_map) & 3u) ||
        (reinterpret_cast<uintptr_t>(recv_src) & 3u) ||
        (reinterpret_cast<uintptr_t>(expert_counts) & 3u))
        return fail(EP_INVALID_ARGUMENT, "int32 outputs and the local map must be 4-byte aligned");
    if ((reinterpret_cast<uintptr_t>(recv_topk_idx) & 7u))
        return fail(EP_INVALID_ARGUMENT, "recv_topk_idx must be 8-byte aligned");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(EP_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    const size_t need = ep_rank_layout_workspace_size(tokens_per_rank, num_experts, num_ranks);
    if (workspace_bytes < need)
        return fail(EP_INVALID_ARGUMENT, "workspace %zu bytes < %zu required", workspace_bytes, need);
    return from_hip(ep::launch_rank_layout(global_routing_map, tokens_per_rank, num_experts,
                                           num_ranks, rank, k_out, sparse_to_dense_map,
                                           local_expert_routing_map, recv_src, recv_topk_idx,
                                           expert_counts, num_recv, num_overflow, workspace,
                                           static_cast<hipStream_t>(stream)),
                    "ep_rank_layout launch");
}

ep_status_t ep_dispatch_ranked(const void* x, const int64_t* topk_idx, const float* topk_weights,
                               int64_t num_tokens, int hidden, int num_topk, int num_experts,
                               int num_ranks, const int32_t* sparse_to_dense_map,
                               void* const* dest_x, float* const* dest_weights, int64_t dest_rows,
                               void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 8);
    if (st) return st;
    st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    if (dest_rows < 0) return fail(EP_INVALID_ARGUMENT, "dest_rows < 0");
    if (!dest_x) return fail(EP_INVALID_ARGUMENT, "dest_x (a host array of pointers) is required");
    ep::RankPtrs px = {}, pw = {};
    for (int d = 0; d < num_ranks; ++d) {
        if (!dest_x[d] || !aligned16(dest_x[d]))
            return fail(EP_INVALID_ARGUMENT, "dest_x[%d] must be non-NULL and 16-byte aligned", d);
        px.p[d] = dest_x[d];
        if (dest_weights) {
            if ((reinterpret_cast<uintptr_t>(dest_weights[d]) & 3u))
                return fail(EP_INVALID_ARGUMENT, "dest_weights[%d] must be 4-byte aligned", d);
            pw.p[d] = dest_weights[d];
        }
    }
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x || !sparse_to_dense_map)
        return fail(EP_INVALID_ARGUMENT, "x and sparse_to_dense_map are required");
    if (!aligned16(x)) return fail(EP_INVALID_ARGUMENT, "x must be 16-byte aligned");
    if (dest_weights && (!topk_idx || (reinterpret_cast<uintptr_t>(topk_idx) & 7u)))
        return fail(EP_INVALID_ARGUMENT, "dest_weights needs an 8-byte aligned topk_idx");
    const ep::RankPtrs none = {};
    return from_hip(ep::launch_dispatch_ranked(x, topk_idx, topk_weights, num_tokens, hidden * 2,
                                               num_topk, num_experts, num_ranks,
                                               sparse_to_dense_map, px, pw, dest_weights != nullptr,
                                               nullptr, none, 0, dest_rows,
                                               static_cast<hipStream_t>(stream)),
                    "ep_dispatch_ranked launch");
}

ep_status_t ep_dispatch_ranked_prequantized(const void* x_q, const float* x_scales,
                                            const int64_t* topk_idx, const float* topk_weights,
                                            int64_t num_tokens, int hidden, int num_topk,
                                            int num_experts, int num_ranks,
                                            const int32_t* sparse_to_dense_map, void* const* dest_q,
                                            float* const* dest_scales, float* const* dest_weights,
                                            int64_t dest_rows, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_hidden(hidden, 128);
    if (st) return st;
    st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    if (dest_rows < 0) return fail(EP_INVALID_ARGUMENT, "dest_rows < 0");
    if (!dest_q || !dest_scales)
        return fail(EP_INVALID_ARGUMENT, "dest_q and dest_scales (host arrays of pointers) are required");
    ep::RankPtrs pq = {}, ps = {}, pw = {};
    for (int d = 0; d < num_ranks; ++d) {
        if (!dest_q[d] || !aligned16(dest_q[d]))
            return fail(EP_INVALID_ARGUMENT, "dest_q[%d] must be non-NULL and 16-byte aligned", d);
        if (!dest_scales[d] || (reinterpret_cast<uintptr_t>(dest_scales[d]) & 3u))
            return fail(EP_INVALID_ARGUMENT, "dest_scales[%d] must be non-NULL and 4-byte aligned", d);
        pq.p[d] = dest_q[d];
        ps.p[d] = dest_scales[d];
        if (dest_weights) {
            if ((reinterpret_cast<uintptr_t>(dest_weights[d]) & 3u))
                return fail(EP_INVALID_ARGUMENT, "dest_weights[%d] must be 4-byte aligned", d);
            pw.p[d] = dest_weights[d];
        }
    }
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x_q || !x_scales || !sparse_to_dense_map)
        return fail(EP_INVALID_ARGUMENT, "x_q, x_scales and sparse_to_dense_map are required");
    if (!aligned16(x_q)) return fail(EP_INVALID_ARGUMENT, "x_q must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(x_scales) & 3u))
        return fail(EP_INVALID_ARGUMENT, "x_scales must be 4-byte aligned");
    if (dest_weights && (!topk_idx || (reinterpret_cast<uintptr_t>(topk_idx) & 7u)))
        return fail(EP_INVALID_ARGUMENT, "dest_weights needs an 8-byte aligned topk_idx");
    return from_hip(ep::launch_dispatch_ranked(x_q, topk_idx, topk_weights, num_tokens, hidden,
                                               num_topk, num_experts, num_ranks,
                                               sparse_to_dense_map, pq, pw, dest_weights != nullptr,
                                               x_scales, ps, hidden / 128, dest_rows,
                                               static_cast<hipStream_t>(stream)),
                    "ep_dispatch_ranked_prequantized launch");
}

ep_status_t ep_dispatch_ranked_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                                   int64_t num_tokens, int hidden, int num_topk, int num_experts,
                                   int num_ranks, const int32_t* sparse_to_dense_map,
                                   int out_dtype, int scale_format, void* const* dest_q,
                                   void* const* dest_scales, float* const* dest_weights,
                                   int64_t dest_rows, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    if (out_dtype != EP_OUT_FP8_E4M3 && out_dtype != EP_OUT_FP8_E5M2)
        return fail(EP_INVALID_ARGUMENT, "out_dtype %d is not an 8-bit format", out_dtype);
    if (scale_format != EP_SCALE_FP32 && scale_format != EP_SCALE_FP32_POW2 &&
        scale_format != EP_SCALE_UE8M0)
        return fail(EP_INVALID_ARGUMENT, "unknown scale_format %d", scale_format);
    st = check_hidden(hidden, 128);
    if (st) return st;
    st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    if (dest_rows < 0) return fail(EP_INVALID_ARGUMENT, "dest_rows < 0");
    if (ep::ranked_fp8_blocks(num_tokens, hidden, num_ranks) > INT32_MAX)
        return fail(EP_UNSUPPORTED, "num_tokens too large for hidden %d and %d ranks", hidden,
                    num_ranks);
    if (!dest_q || !dest_scales)
        return fail(EP_INVALID_ARGUMENT, "dest_q and dest_scales (host arrays of pointers) are required");
    const bool bytes = scale_format == EP_SCALE_UE8M0;
    ep::RankPtrs pq = {}, ps = {}, pw = {};
    for (int d = 0; d < num_ranks; ++d) {
        if (!dest_q[d] || !aligned16(dest_q[d]))
            return fail(EP_INVALID_ARGUMENT, "dest_q[%d] must be non-NULL and 16-byte aligned", d);
        if (!dest_scales[d] || (!bytes && (reinterpret_cast<uintptr_t>(dest_scales[d]) & 3u)))
            return fail(EP_INVALID_ARGUMENT, "dest_scales[%d] must be non-NULL%s", d,
                        bytes ? "" : " and 4-byte aligned");
        pq.p[d] = dest_q[d];
        ps.p[d] = dest_scales[d];
        if (dest_weights) {
            if ((reinterpret_cast<uintptr_t>(dest_weights[d]) & 3u))
                return fail(EP_INVALID_ARGUMENT, "dest_weights[%d] must be 4-byte aligned", d);
            pw.p[d] = dest_weights[d];
        }
    }
    if (num_tokens == 0) return EP_SUCCESS;
    if (!x || !sparse_to_dense_map)
        return fail(EP_INVALID_ARGUMENT, "x and sparse_to_dense_map are required");
    if (!aligned16(x)) return fail(EP_INVALID_ARGUMENT, "x must be 16-byte aligned");
    if (dest_weights && (!topk_idx || (reinterpret_cast<uintptr_t>(topk_idx) & 7u)))
        return fail(EP_INVALID_ARGUMENT, "dest_weights needs an 8-byte aligned topk_idx");
    return from_hip(ep::launch_dispatch_ranked_fp8(x, topk_idx, topk_weights, num_tokens, hidden,
                                                   num_topk, num_experts, num_ranks,
                                                   sparse_to_dense_map,
                                                   out_dtype == EP_OUT_FP8_E5M2 ? 1 : 0,
                                                   scale_format, pq, ps, pw,
                                                   dest_weights != nullptr, dest_rows,
                                                   static_cast<hipStream_t>(stream)),
                    "ep_dispatch_ranked_fp8 launch");
}

// Checks shared by the two fused-permute entry points; fills the pointer
// tables (src_s only when scales is true).
static ep_status_t fused_permute_args(const void* const* src_x, const float* const* src_s,
                                      bool scales, const int64_t* const* src_topk_idx,
                                      const float* const* src_topk_weights,
                                      int64_t tokens_per_rank, int hidden, int hidden_multiple,
                                      int num_topk, int num_experts, int num_ranks, int rank,
                                      int64_t rows, float* recv_weights, ep::RankPtrs& px,
                                      ep::RankPtrs& ps, ep::RankPtrs& pi, ep::RankPtrs& pw)
{
    if (tokens_per_rank < 0) return fail(EP_INVALID_ARGUMENT, "tokens_per_rank < 0");
    ep_status_t st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    st = check_tokens(tokens_per_rank * num_ranks, num_topk);
    if (st) return st;
    st = check_hidden(hidden, hidden_multiple);
    if (st) return st;
    if (rank < 0 || rank >= num_ranks)
        return fail(EP_INVALID_ARGUMENT, "rank %d outside [0, %d)", rank, num_ranks);
    if (rows < 0) return fail(EP_INVALID_ARGUMENT, "rows < 0");
    if (tokens_per_rank == 0) return EP_SUCCESS;   // nothing is read or written
    if (!src_x) return fail(EP_INVALID_ARGUMENT, "src_x (a host array of pointers) is required");
    if (scales && !src_s)
        return fail(EP_INVALID_ARGUMENT, "src_scales (a host array of pointers) is required");
    if (recv_weights && !src_topk_idx)
        return fail(EP_INVALID_ARGUMENT, "recv_weights needs src_topk_idx");
    for (int d = 0; d < num_ranks; ++d) {
        if (!src_x[d] || !aligned16(src_x[d]))
            return fail(EP_INVALID_ARGUMENT, "src_x[%d] must be non-NULL and 16-byte aligned", d);
        px.p[d] = const_cast<void*>(src_x[d]);
        if (scales) {
            if (!src_s[d] || (reinterpret_cast<uintptr_t>(src_s[d]) & 3u))
                return fail(EP_INVALID_ARGUMENT,
                            "src_scales[%d] must be non-NULL and 4-byte aligned", d);
            ps.p[d] = const_cast<float*>(src_s[d]);
        }
        if (recv_weights) {
            if (!src_topk_idx[d] || (reinterpret_cast<uintptr_t>(src_topk_idx[d]) & 7u))
                return fail(EP_INVALID_ARGUMENT,
                            "src_topk_idx[%d] must be non-NULL and 8-byte aligned", d);
            pi.p[d] = const_cast<int64_t*>(src_topk_idx[d]);
            if (src_topk_weights) {
                if ((reinterpret_cast<uintptr_t>(src_topk_weights[d]) & 3u))
                    return fail(EP_INVALID_ARGUMENT, "src_topk_weights[%d] must be 4-byte aligned",
                                d);
                pw.p[d] = const_cast<float*>(src_topk_weights[d]);
            }
        }
    }
    return EP_SUCCESS;
}

static ep_status_t fused_permute_outputs(const int32_t* recv_src, const int32_t* slot,
                                         const void* recv_x, const int64_t* recv_topk_idx,
                                         const float* recv_weights, const int32_t* num_recv)
{
    if (!recv_src || !slot || !recv_x || (recv_weights && !recv_topk_idx))
        return fail(EP_INVALID_ARGUMENT,
                    "recv_src, slot, recv_x (and recv_topk_idx with recv_weights) are required");
    if (!aligned16(recv_x)) return fail(EP_INVALID_ARGUMENT, "recv_x must be 16-byte aligned");
    if (num_recv && (reinterpret_cast<uintptr_t>(num_recv) & 3u))
        return fail(EP_INVALID_ARGUMENT, "num_recv must be 4-byte aligned");
    return EP_SUCCESS;
}

ep_status_t ep_dispatch_fused_permute(const void* const* src_x, const int64_t* const* src_topk_idx,
                                      const float* const* src_topk_weights, int64_t tokens_per_rank,
                                      int hidden, int num_topk, int num_experts, int num_ranks,
                                      int rank, const int32_t* recv_src,
                                      const int64_t* recv_topk_idx, const int32_t* num_recv,
                                      const int32_t* slot, int64_t rows, void* recv_x,
                                      float* recv_weights, void* stream)
{
    g_last_error[0] = '\0';
    ep::RankPtrs px = {}, ps = {}, pi = {}, pw = {};
    ep_status_t st = fused_permute_args(src_x, nullptr, false, src_topk_idx, src_topk_weights,
                                        tokens_per_rank, hidden, 8, num_topk, num_experts,
                                        num_ranks, rank, rows, recv_weights, px, ps, pi, pw);
    if (st) return st;
    if (tokens_per_rank == 0) return EP_SUCCESS;
    st = fused_permute_outputs(recv_src, slot, recv_x, recv_topk_idx, recv_weights, num_recv);
    if (st) return st;
    return from_hip(ep::launch_dispatch_fused_permute(px, pi, pw, tokens_per_rank, hidden, num_topk,
                                                      num_experts, num_ranks, rank, recv_src,
                                                      recv_topk_idx, num_recv, slot, rows, recv_x,
                                                      recv_weights, static_cast<hipStream_t>(stream)),
                    "ep_dispatch_fused_permute launch");
}

ep_status_t ep_dispatch_fused_permute_prequantized(
    const void* const* src_q, const float* const* src_scales, const int64_t* const* src_topk_idx,
    const float* const* src_topk_weights, int64_t tokens_per_rank, int hidden, int num_topk,
    int num_experts, int num_ranks, int rank, const int32_t* recv_src,
    const int64_t* recv_topk_idx, const int32_t* num_recv, const int32_t* slot, int64_t rows,
    void* recv_q, float* recv_scales, float* recv_weights, void* stream)
{
    g_last_error[0] = '\0';
    ep::RankPtrs px = {}, ps = {}, pi = {}, pw = {};
    ep_status_t st = fused_permute_args(src_q, src_scales, true, src_topk_idx, src_topk_weights,
                                        tokens_per_rank, hidden, 128, num_topk, num_experts,
                                        num_ranks, rank, rows, recv_weights, px, ps, pi, pw);
    if (st) return st;
    if (tokens_per_rank == 0) return EP_SUCCESS;
    st = fused_permute_outputs(recv_src, slot, recv_q, recv_topk_idx, recv_weights, num_recv);
    if (st) return st;
    if (!recv_scales || (reinterpret_cast<uintptr_t>(recv_scales) & 3u))
        return fail(EP_INVALID_ARGUMENT, "recv_scales must be non-NULL and 4-byte aligned");
    return from_hip(ep::launch_dispatch_fused_permute_prequant(
                        px, ps, pi, pw, tokens_per_rank, hidden, num_topk, num_experts, num_ranks,
                        rank, recv_src, recv_topk_idx, num_recv, slot, rows, recv_q, recv_scales,
                        recv_weights, static_cast<hipStream_t>(stream)),
                    "ep_dispatch_fused_permute_prequantized launch");
}

ep_status_t ep_combine_ranked(const void* const* src_y, int64_t src_rows,
                              const int32_t* sparse_to_dense_map, int64_t num_tokens, int hidden,
                              int num_ranks, void* out, void* stream)
{
    g_last_error[0] = '\0';
    if (num_tokens < 0) return fail(EP_INVALID_ARGUMENT, "num_tokens < 0");
    if (num_ranks < 1 || num_ranks > EP_MAX_RANKS)
        return fail(EP_INVALID_ARGUMENT, "num_ranks %d outside [1, %d]", num_ranks, EP_MAX_RANKS);
    if (num_tokens * (int64_t)num_ranks >= ((int64_t)1 << 31))
        return fail(EP_UNSUPPORTED, "num_tokens * num_ranks must be < 2^31");
    ep_status_t st = check_hidden(hidden, 8);
    if (st) return st;
    if (src_rows < 0) return fail(EP_INVALID_ARGUMENT, "src_rows < 0");
    if (!src_y) return fail(EP_INVALID_ARGUMENT, "src_y (a host array of pointers) is required");
    ep::RankPtrs ps = {};
    for (int d = 0; d < num_ranks; ++d) {
        if (!src_y[d] || !aligned16(src_y[d]))
            return fail(EP_INVALID_ARGUMENT, "src_y[%d] must be non-NULL and 16-byte aligned", d);
        ps.p[d] = const_cast<void*>(src_y[d]);
    }
    if (num_tokens == 0) return EP_SUCCESS;
    if (!sparse_to_dense_map || !out)
        return fail(EP_INVALID_ARGUMENT, "sparse_to_dense_map and out are required");
    if (!aligned16(out)) return fail(EP_INVALID_ARGUMENT, "out must be 16-byte aligned");
    return from_hip(ep::launch_combine_ranked(ps, src_rows, sparse_to_dense_map, num_tokens, hidden,
                                              num_ranks, out, static_cast<hipStream_t>(stream)),
                    "ep_combine_ranked launch");
}

ep_status_t ep_dispatch_ranked_backward(const void* const* grad_recv_x,
                                        const float* const* grad_recv_weights, int64_t src_rows,
                                        const int64_t* topk_idx, const int32_t* sparse_to_dense_map,
                                        int64_t num_tokens, int hidden, int num_topk,
                                        int num_experts, int num_ranks, void* grad_x,
                                        float* grad_topk_weights, void* stream)
{
    g_last_error[0] = '\0';
    ep_status_t st = check_tokens(num_tokens, num_topk);
    if (st) return st;
    st = check_ranks(num_experts, num_ranks);
    if (st) return st;
    if (num_tokens * (int64_t)num_ranks >= ((int64_t)1 << 31))
        return fail(EP_UNSUPPORTED, "num_tokens * num_ranks must be < 2^31");
    if (src_rows < 0) return fail(EP_INVALID_ARGUMENT, "src_rows < 0");
    if (!grad_recv_x && !grad_recv_weights)
        return fail(EP_INVALID_ARGUMENT, "nothing to do: grad_recv_x and grad_recv_weights are NULL");
    if ((grad_recv_x != nullptr) != (grad_x != nullptr))
        return fail(EP_INVALID_ARGUMENT, "grad_recv_x and grad_x go together");
    if ((grad_recv_weights != nullptr) != (grad_topk_weights != nullptr))
        return fail(EP_INVALID_ARGUMENT, "grad_recv_weights and grad_topk_weights go together");
    ep::RankPtrs px = {}, pw = {};
    if (grad_recv_x) {
        st = check_hidden(hidden, 8);
        if (st) return st;
        for (int d = 0; d < num_ranks; ++d) {
            if (!grad_recv_x[d] || !aligned16(grad_recv_x[d]))
                return fail(EP_INVALID_ARGUMENT, "grad_recv_x[%d] must be non-NULL and 16-byte aligned",
                            d);
            px.p[d] = const_cast<void*>(grad_recv_x[d]);
        }
        if (num_tokens > 0 && !aligned16(grad_x))
            return fail(EP_INVALID_ARGUMENT, "grad_x must be 16-byte aligned");
    }
    if (grad_recv_weights) {
        for (int d = 0; d < num_ranks; ++d) {
            if ((reinterpret_cast<uintptr_t>(grad_recv_weights[d]) & 3u))
                return fail(EP_INVALID_ARGUMENT, "grad_recv_weights[%d] must be 4-byte aligned", d);
            pw.p[d] = const_cast<float*>(grad_recv_weights[d]);
        }
        if (num_tokens > 0 && (!topk_idx || (reinterpret_cast<uintptr_t>(topk_idx) & 7u)))
            return fail(EP_INVALID_ARGUMENT, "grad_recv_weights needs an 8-byte aligned topk_idx");
        if (num_tokens > 0 && (reinterpret_cast<uintptr_t>(grad_topk_weights) & 3u))
            return fail(EP_INVALID_ARGUMENT, "grad_topk_weights must be 4-byte aligned");
    }
    if (num_tokens == 0) return EP_SUCCESS;
    if (!sparse_to_dense_map) return fail(EP_INVALID_ARGUMENT, "sparse_to_dense_map is required");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (grad_recv_x) {
        st = from_hip(ep::launch_combine_ranked(px, src_rows, sparse_to_dense_map, num_tokens,
                                                hidden, num_ranks, grad_x, s),
                      "ep_dispatch_ranked_backward launch (tokens)");
        if (st) return st;
    }
    if (grad_recv_weights)
        return from_hip(ep::launch_ranked_weight_grad(pw, src_rows, topk_idx, sparse_to_dense_map,
                                                      num_tokens, num_topk, num_experts, num_ranks,
                                                      grad_topk_weights, s),
                        "ep_dispatch_ranked_backward launch (weights)");
    return EP_SUCCESS;
}

}  // extern "C"

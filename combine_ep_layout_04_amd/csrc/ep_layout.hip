// ep_layout.hip -- routing layout of one device's tokens on gfx950.
//
// What is computed (NCCL EP page, nccl_ep.cc, ncclEpCreateHandle "Step 3"
// metadata preprocessing: per-expert counts of the tokens routed here;
// DeepEP page, "Prefix Sum Interpretation for Expert Token Counts": in the
// expanded layout expert i owns rows [psum[i-1], psum[i]); NeMo fused_a2a
// page, HybridEPDispatch: -1 marks an unused top-k slot):
//
//   counts[e]   number of pairs i = t*k + j with topk_idx[i] == e
//   offsets[e]  exclusive prefix sum of counts (offsets[E] = N)
//   slot[i]     offsets[e] + #{i' < i : topk_idx[i'] == e}, or -1
//   src[r]      the token t of the pair whose slot is r
//
// The pages' preprocessing counts with atomics; here atomics only ever
// produce counts, never positions, so the result is a deterministic stable
// counting sort.  Three launches, each linear in the number of pairs:
//
//   1. count:   one workgroup per chunk of kLayoutChunk pairs builds the
//               chunk's expert histogram in LDS -> hist[c][e].
//   2. scan:    one workgroup of 1024 threads turns hist into per-(chunk,
//               expert) starting rows in place (column running sums over
//               chunks plus the exclusive scan over experts) and writes
//               counts / offsets.
//   3. scatter: each chunk again, in batches of 256 pairs.  Inside a batch
//               every pair sets its bit in an LDS bit-matrix row of its
//               expert (256 bits = 8 words per expert); its rank among
//               earlier pairs of the same expert is a popcount of the bits
//               below its own, so no ordering depends on atomic timing.
//
// The workspace holds hist (C*E int32, rewritten in place by the scan) and
// one invalid-entry count per chunk.

#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMaxExperts = 1024;                 // EP_MAX_EXPERTS
constexpr int kWords = kLayoutThreads / 32;       // bit words per expert per batch
constexpr int kScanThreads = 1024;

static_assert(kLayoutChunk % kLayoutThreads == 0, "chunk must be whole batches");

// Exclusive scan of one int per thread over the workgroup (blockDim a
// multiple of 64).  `waves` is LDS scratch of blockDim/64 ints.  Returns the
// exclusive prefix and writes the workgroup total to *total.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* waves, int32_t* total)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) waves[wave] = x;
    __syncthreads();
    int32_t before = 0, all = 0;
    for (int w = 0; w < nwaves; ++w) {
        const int32_t s = waves[w];
        before += (w < wave) ? s : 0;
        all += s;
    }
    *total = all;
    return before + x - v;
}

__global__ __launch_bounds__(kLayoutThreads)
void layout_count_kernel(const int64_t* __restrict__ idx, int64_t pairs, int E,
                         int32_t* __restrict__ hist, int32_t* __restrict__ bad)
{
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t nbad;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kLayoutThreads) cnt[e] = 0;
    if (tid == 0) nbad = 0;
    __syncthreads();

    const int64_t begin = (int64_t)blockIdx.x * kLayoutChunk;
    const int64_t end = min(begin + (int64_t)kLayoutChunk, pairs);
#pragma unroll 4
    for (int64_t i = begin + tid; i < end; i += kLayoutThreads) {
        const int64_t e = idx[i];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else if (e != -1)
            atomicAdd(&nbad, 1);
    }
    __syncthreads();

    int32_t* h = hist + (int64_t)blockIdx.x * E;
    for (int e = tid; e < E; e += kLayoutThreads) h[e] = cnt[e];
    if (tid == 0) bad[blockIdx.x] = nbad;
}

// hist is C rows (chunks) x E columns (experts).  The 1024 threads tile it:
// epad = E rounded up to a power of two columns, tpc = 1024 / epad threads
// per column, each owning a contiguous slab of rows.  Loads are batched
// kBatch at a time so a thread has one memory round trip per batch, not one
// per row.
constexpr int kBatch = 16;

__global__ __launch_bounds__(kScanThreads)
void layout_scan_kernel(int32_t* __restrict__ hist, const int32_t* __restrict__ bad,
                        int num_chunks, int E, int epad, int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets, int32_t* __restrict__ num_invalid)
{
    __shared__ int32_t part_sum[kScanThreads];
    __shared__ int32_t col_start[kMaxExperts];
    __shared__ int32_t waves[kScanThreads / 64];
    __shared__ int32_t nbad;
    const int tid = threadIdx.x;
    const int tpc = kScanThreads / epad;
    const int col = tid & (epad - 1);
    const int part = tid / epad;
    const int rows = (num_chunks + tpc - 1) / tpc;
    const int r0 = min(part * rows, num_chunks);
    const int r1 = min(r0 + rows, num_chunks);
    const bool live = col < E;
    if (tid == 0) nbad = 0;

    // 1. sum of this thread's slab of its column
    int32_t mine = 0;
    if (live) {
        for (int r = r0; r < r1; r += kBatch) {
            int32_t h[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                h[b] = (r + b < r1) ? hist[(int64_t)(r + b) * E + col] : 0;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) mine += h[b];
        }
    }
    part_sum[tid] = mine;
    __syncthreads();

    // 2. column total, and the rows of this column in earlier slabs
    int32_t before = 0, tot = 0;
    for (int q = 0; q < tpc; ++q) {
        const int32_t v = part_sum[col + q * epad];
        before += (q < part) ? v : 0;
        tot += v;
    }
    // 3. exclusive scan of column totals over experts: the part-0 threads
    // are tids 0..epad-1, in column order, and everyone else adds 0
    int32_t n = 0;
    const int32_t start = block_exclusive_scan((part == 0 && live) ? tot : 0, waves, &n);
    if (part == 0) col_start[col] = start;
    __syncthreads();

    // 4. rewrite the slab in place with each (chunk, expert)'s first row
    if (live) {
        int32_t run = col_start[col] + before;
        for (int r = r0; r < r1; r += kBatch) {
            int32_t h[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                h[b] = (r + b < r1) ? hist[(int64_t)(r + b) * E + col] : 0;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (r + b < r1) hist[(int64_t)(r + b) * E + col] = run;
                run += h[b];
            }
        }
        if (part == 0) {
            counts[col] = tot;
            offsets[col] = start;
        }
    }
    if (tid == 0) offsets[E] = n;

    if (num_invalid) {
        int32_t b = 0;
        for (int c = tid; c < num_chunks; c += kScanThreads) b += bad[c];
        if (b) atomicAdd(&nbad, b);
        __syncthreads();
        if (tid == 0) *num_invalid = nbad;
    }
}

__global__ __launch_bounds__(kLayoutThreads)
void layout_scatter_kernel(const int64_t* __restrict__ idx, int64_t pairs, int k, int E,
                           const int32_t* __restrict__ start, int32_t* __restrict__ slot,
                           int32_t* __restrict__ src)
{
    __shared__ int32_t base[kMaxExperts];
    __shared__ uint32_t bits[kMaxExperts * kWords];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;

    const int32_t* s = start + c * E;
    for (int e = tid; e < E; e += kLayoutThreads) base[e] = s[e];
    for (int w = tid; w < E * kWords; w += kLayoutThreads) bits[w] = 0;
    __syncthreads();

    const int64_t begin = c * kLayoutChunk;
    const int64_t end = min(begin + (int64_t)kLayoutChunk, pairs);
    const int word = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);

    for (int64_t b0 = begin; b0 < end; b0 += kLayoutThreads) {
        const int64_t i = b0 + tid;
        const bool live = i < end;
        const int64_t e64 = live ? idx[i] : -1;
        const bool ok = e64 >= 0 && e64 < E;
        const int e = ok ? (int)e64 : 0;
        if (ok) atomicOr(&bits[e * kWords + word], bit);
        __syncthreads();

        int rank = 0, tot = 0;
        if (ok) {
            const uint32_t* row = &bits[e * kWords];
#pragma unroll
            for (int q = 0; q < kWords; ++q) {
                const uint32_t m = row[q];
                const int pc = __popc(m);
                tot += pc;
                rank += (q < word) ? pc : (q == word ? __popc(m & (bit - 1u)) : 0);
            }
            const int32_t r = base[e] + rank;
            slot[i] = r;
            if (src) src[r] = (int32_t)i / k;
        } else if (live) {
            slot[i] = -1;
        }
        __syncthreads();

        if (ok) {
            if (rank == tot - 1) base[e] += tot;   // the batch's last pair of e
            bits[e * kWords + word] = 0;
        }
        __syncthreads();
    }
}

}  // namespace

int64_t layout_num_chunks(int64_t pairs)
{
    return pairs <= 0 ? 1 : (pairs + kLayoutChunk - 1) / kLayoutChunk;
}

size_t layout_workspace_bytes(int64_t pairs, int num_experts)
{
    const int64_t C = layout_num_chunks(pairs);
    const size_t bytes = (size_t)(C * (int64_t)num_experts + C) * sizeof(int32_t);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                         int num_experts, int32_t* counts, int32_t* offsets, int32_t* slot,
                         int32_t* src, int32_t* num_invalid, void* workspace,
                         hipStream_t stream)
{
    const int64_t pairs = num_tokens * (int64_t)num_topk;
    const int64_t C = layout_num_chunks(pairs);
    int32_t* hist = static_cast<int32_t*>(workspace);
    int32_t* bad = hist + C * num_experts;

    hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)C), dim3(kLayoutThreads), 0, stream,
                       topk_idx, pairs, num_experts, hist, bad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    int epad = 1;
    while (epad < num_experts) epad <<= 1;
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                       hist, bad, (int)C, num_experts, epad, counts, offsets, num_invalid);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    if (pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(layout_scatter_kernel, dim3((unsigned)C), dim3(kLayoutThreads), 0, stream,
                       topk_idx, pairs, num_topk, num_experts, hist, slot, src);
    return hipGetLastError();
}

}  // namespace ep

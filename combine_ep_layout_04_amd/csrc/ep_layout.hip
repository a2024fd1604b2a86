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
// counting sort.  Inputs of up to kLayoutSmallMaxPairs pairs (and at most
// 256 experts) take one launch (layout_single_kernel, described with it);
// larger ones two launches, each linear in the number of pairs:
//
//   1. count:   one workgroup per chunk of pairs (about 64 chunks of at
//               least 256 pairs for small inputs; 1024, or more once there
//               would be over 256 chunks, for large ones) builds the
//               chunk's expert histogram in LDS and writes it transposed,
//               hist[e][c], with the chunk count padded to a multiple of 4
//               (padding chunks are empty and write zeros).
//   2. scatter: each workgroup first derives what it needs from the whole
//               histogram -- every expert's total (for offsets) and its rows
//               in earlier chunks -- reading each expert's chunk counts as
//               16-byte vectors; workgroup 0 also writes counts, offsets and
//               num_invalid.  Then it ranks its chunk's pairs.  Up to 256
//               experts (layout_scatter_wide_kernel): 1024 lanes, 1024 pairs
//               at a time, a pair's rank within its wavefront found by
//               ballots over its expert id's bits, and per-(wavefront,
//               expert) base rows from an exclusive sum over the
//               wavefronts (at T=8192, k=8, E=256: 6.6 against 8.7 us, the
//               layout 14.0 against 16.1 us by HIP events).  More experts
//               (layout_scatter_kernel): 256 lanes, batches of 256 pairs,
//               every pair setting its bit in an LDS bit-matrix row of its
//               expert (256 bits = 8 words per expert), its rank the
//               popcount of the bits below its own.  Either way no position
//               depends on atomic timing.
//
// Segment placement (DeepEP page, "Prefix Sum Interpretation for Expert
// Token Counts": in expand mode an expert's rows start at
// align(psum[i-1], expert_alignment); NeMo page, HybridEP pad_multiple; NCCL
// EP page, ncclEpDispatch low-latency branch: recv_x [experts, capacity,
// hidden] with per-expert receive counts):
//   packed       start[e] = sum_{e'<e} align_up(count[e'], alignment)
//   fixed stride start[e] = e * capacity; pairs whose rank within their
//                expert reaches the capacity are dropped (slot -1) and
//                counted, so nothing is ever written past the buffer.
//
// The workspace holds hist (E * Cp int32) and one invalid-entry count per
// chunk.  Folding the scan into the scatter saves a launch: at 64 chunks the
// redundant per-workgroup reads are 64 KiB from L2 each.

#include <algorithm>
#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMaxExperts = 1024;                 // EP_MAX_EXPERTS
constexpr int kWords = kLayoutThreads / 32;       // bit words per expert per batch
// LDS row stride of the bit matrix: one word of padding makes it odd, so
// the rows of different experts start in different banks (a stride of 8
// words put 64 lanes with random experts on 8 of the 32 banks)
constexpr int kRowStride = kWords + 1;

static_assert(kLayoutMinChunk % kLayoutThreads == 0, "chunk must be whole batches");

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
void layout_count_kernel(const int64_t* __restrict__ idx, int64_t pairs, int64_t chunk, int E,
                         int cpad, int32_t* __restrict__ hist, int32_t* __restrict__ bad)
{
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t nbad;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kLayoutThreads) cnt[e] = 0;
    if (tid == 0) nbad = 0;
    __syncthreads();

    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = min(begin + chunk, pairs);
#pragma unroll 4
    for (int64_t i = begin + tid; i < end; i += kLayoutThreads) {
        const int64_t e = idx[i];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else if (e != -1)
            atomicAdd(&nbad, 1);
    }
    __syncthreads();

    for (int e = tid; e < E; e += kLayoutThreads) hist[(int64_t)e * cpad + blockIdx.x] = cnt[e];
    if (tid == 0) bad[blockIdx.x] = nbad;
}

// Sum of n int32 at p (16-byte aligned, n a multiple of 4), and the sum of
// the first `upto` of them.
__device__ __forceinline__ void sum_row(const int32_t* p, int n, int upto, int32_t& all,
                                        int32_t& before)
{
    const int4* v = reinterpret_cast<const int4*>(p);
    int32_t a = 0, b = 0;
    for (int i0 = 0; i0 < n / 4; i0 += 8) {
        int4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = (i0 + u < n / 4) ? v[i0 + u] : make_int4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int c = 4 * (i0 + u);
            a += q[u].x + q[u].y + q[u].z + q[u].w;
            b += (c < upto ? q[u].x : 0) + (c + 1 < upto ? q[u].y : 0) +
                 (c + 2 < upto ? q[u].z : 0) + (c + 3 < upto ? q[u].w : 0);
        }
    }
    all = a;
    before = b;
}

__global__ __launch_bounds__(kLayoutThreads)
void layout_scatter_kernel(const int64_t* __restrict__ idx, int64_t pairs, int64_t chunk, int k,
                           int E, int cpad, int num_chunks, int alignment, int capacity,
                           const int32_t* __restrict__ hist, const int32_t* __restrict__ bad,
                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ slot, int32_t* __restrict__ src,
                           int32_t* __restrict__ num_invalid, int32_t* __restrict__ num_dropped)
{
    __shared__ int32_t base[kMaxExperts];
    __shared__ int32_t total[kMaxExperts];
    __shared__ int32_t seg[kMaxExperts];
    __shared__ int32_t ndrop;
    __shared__ uint32_t bits[kMaxExperts * kRowStride];
    __shared__ int32_t waves[kLayoutThreads / 64];
    __shared__ int32_t nbad;
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;

    // 1. every expert's total and its rows in chunks before this one
    for (int e = tid; e < E; e += kLayoutThreads) {
        int32_t all, before;
        sum_row(hist + (int64_t)e * cpad, cpad, (int)c, all, before);
        total[e] = all;
        base[e] = before;
    }
    for (int w = tid; w < E * kRowStride; w += kLayoutThreads) bits[w] = 0;
    if (tid == 0) nbad = 0;
    __syncthreads();

    // 2. segment starts: packed segments are an exclusive scan of the counts
    // rounded up to the alignment (thread t owns the contiguous experts
    // [t*per, t*per + per)); fixed-stride segments start at e * capacity
    const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
    int32_t local = 0;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < E) local += (total[e] + alignment - 1) / alignment * alignment;
    }
    int32_t n = 0;
    int32_t run = block_exclusive_scan(local, waves, &n);
    if (tid == 0) ndrop = 0;
    int32_t drop = 0;
    for (int q = 0; q < per; ++q) {
        const int e = tid * per + q;
        if (e < E) {
            const int32_t tot = total[e];
            const int32_t start = capacity > 0 ? e * capacity : run;
            seg[e] = start;
            base[e] += start;
            if (c == 0) {
                counts[e] = capacity > 0 ? min(tot, capacity) : tot;
                offsets[e] = start;
            }
            if (capacity > 0 && tot > capacity) drop += tot - capacity;
            run += (tot + alignment - 1) / alignment * alignment;
        }
    }
    if (c == 0) {
        if (tid == 0) offsets[E] = capacity > 0 ? E * capacity : n;
        if (num_invalid) {
            int32_t b = 0;
            for (int cc = tid; cc < num_chunks; cc += kLayoutThreads) b += bad[cc];
            if (b) atomicAdd(&nbad, b);
        }
    }
    __syncthreads();
    if (c == 0 && num_dropped && drop) atomicAdd(&ndrop, drop);
    __syncthreads();
    if (c == 0 && tid == 0) {
        if (num_invalid) *num_invalid = nbad;
        if (num_dropped) *num_dropped = ndrop;
    }

    const int64_t begin = c * chunk;
    const int64_t end = min(begin + chunk, pairs);
    const int word = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);

    for (int64_t b0 = begin; b0 < end; b0 += kLayoutThreads) {
        const int64_t i = b0 + tid;
        const bool live = i < end;
        const int64_t e64 = live ? idx[i] : -1;
        const bool ok = e64 >= 0 && e64 < E;
        const int e = ok ? (int)e64 : 0;
        if (ok) atomicOr(&bits[e * kRowStride + word], bit);
        __syncthreads();

        int rank = 0, tot = 0;
        if (ok) {
            const uint32_t* row = &bits[e * kRowStride];
#pragma unroll
            for (int q = 0; q < kWords; ++q) {
                const uint32_t m = row[q];
                const int pc = __popc(m);
                tot += pc;
                rank += (q < word) ? pc : (q == word ? __popc(m & (bit - 1u)) : 0);
            }
            const int32_t r = base[e] + rank;
            if (capacity > 0 && r - seg[e] >= capacity) {
                slot[i] = -1;                       // past the expert's capacity
            } else {
                slot[i] = r;
                if (src) src[r] = (int32_t)i / k;
            }
        } else if (live) {
            slot[i] = -1;
        }
        __syncthreads();

        if (ok) {
            if (rank == tot - 1) base[e] += tot;   // the batch's last pair of e
            bits[e * kRowStride + word] = 0;
        }
        __syncthreads();
    }
}

// Wide scatter, for at most kWideMaxExperts experts: the same result as
// layout_scatter_kernel from workgroups of 16 wavefronts, which take their
// chunk 1024 pairs at a time (one per lane) and rank them without a bit
// matrix: within a wavefront, the lanes holding the same expert are found
// by ballots over the id's bits (the popcount of the lower ones is a pair's
// rank there), each wavefront's per-expert count is written by that
// expert's lowest lane, and an exclusive sum over the wavefronts, per
// expert, gives every (wavefront, expert) base row.  Four lanes share each
// expert's histogram row in the prologue.
constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / 64;
constexpr int kWideMaxExperts = 256;

__global__ __launch_bounds__(kWideThreads)
void layout_scatter_wide_kernel(const int64_t* __restrict__ idx, int64_t pairs, int64_t chunk, int k,
                                int E, int cpad, int num_chunks, int alignment, int capacity,
                                const int32_t* __restrict__ hist, const int32_t* __restrict__ bad,
                                int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                int32_t* __restrict__ slot, int32_t* __restrict__ src,
                                int32_t* __restrict__ num_invalid, int32_t* __restrict__ num_dropped)
{
    __shared__ int32_t base[kWideMaxExperts];
    __shared__ int32_t total[kWideMaxExperts];
    __shared__ int32_t seg[kWideMaxExperts];
    __shared__ int32_t wcnt[kWideWaves][kWideMaxExperts];
    __shared__ int32_t waves[kWideWaves];
    __shared__ int32_t nbad, ndrop;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int64_t c = blockIdx.x;

    // 1. every expert's total and its rows in earlier chunks: lanes 4e..4e+3
    // each sum a quarter of expert e's histogram row (16-byte vectors)
    {
        const int e = tid >> 2, part = tid & 3;
        int32_t a = 0, b = 0;
        if (e < E) {
            const int nv = cpad / 4;
            const int4* v = reinterpret_cast<const int4*>(hist + (int64_t)e * cpad);
            for (int q = part; q < nv; q += 4) {
                const int4 h = v[q];
                const int c0 = 4 * q;
                a += h.x + h.y + h.z + h.w;
                b += (c0 < c ? h.x : 0) + (c0 + 1 < c ? h.y : 0) + (c0 + 2 < c ? h.z : 0) +
                     (c0 + 3 < c ? h.w : 0);
            }
        }
        a += __shfl_xor(a, 1, 64);
        b += __shfl_xor(b, 1, 64);
        a += __shfl_xor(a, 2, 64);
        b += __shfl_xor(b, 2, 64);
        if (e < E && part == 0) {
            total[e] = a;
            base[e] = b;
        }
    }
    if (tid == 0) {
        nbad = 0;
        ndrop = 0;
    }
    __syncthreads();

    // 2. segment starts (thread e owns expert e)
    const int32_t tot = tid < E ? total[tid] : 0;
    const int32_t padded = tid < E ? (tot + alignment - 1) / alignment * alignment : 0;
    int32_t n = 0;
    const int32_t run = block_exclusive_scan(padded, waves, &n);
    if (tid < E) {
        const int32_t start = capacity > 0 ? tid * capacity : run;
        seg[tid] = start;
        base[tid] += start;
        if (c == 0) {
            counts[tid] = capacity > 0 ? min(tot, capacity) : tot;
            offsets[tid] = start;
            if (capacity > 0 && tot > capacity) atomicAdd(&ndrop, tot - capacity);
        }
    }
    if (c == 0) {
        if (tid == 0) offsets[E] = capacity > 0 ? E * capacity : n;
        if (num_invalid) {
            int32_t bb = 0;
            for (int cc = tid; cc < num_chunks; cc += kWideThreads) bb += bad[cc];
            if (bb) atomicAdd(&nbad, bb);
        }
    }
    __syncthreads();
    if (c == 0 && tid == 0) {
        if (num_invalid) *num_invalid = nbad;
        if (num_dropped) *num_dropped = ndrop;
    }

    // 3. the chunk, 1024 pairs at a time
    const int64_t begin = c * chunk;
    const int64_t end = min(begin + chunk, pairs);
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int64_t b0 = begin; b0 < end; b0 += kWideThreads) {
        const int64_t i = b0 + tid;
        const bool live = i < end;
        const int64_t e64 = live ? idx[i] : -1;
        const bool ok = e64 >= 0 && e64 < E;
        const int ex = ok ? (int)e64 : 0;
        uint64_t m = __ballot(ok);
        for (int bt = 0; bt < nbits; ++bt) {
            const bool bit = ok && ((ex >> bt) & 1);
            const uint64_t bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        const uint64_t below = m & ((1ull << lane) - 1ull);
        for (int q = tid; q < kWideWaves * kWideMaxExperts; q += kWideThreads) (&wcnt[0][0])[q] = 0;
        __syncthreads();
        if (ok && below == 0) wcnt[w][ex] = __popcll(m);     // the expert's lowest lane
        __syncthreads();
        if (tid < E) {
            int32_t r = base[tid];
            for (int v = 0; v < kWideWaves; ++v) {
                const int32_t cnt = wcnt[v][tid];
                wcnt[v][tid] = r;
                r += cnt;
            }
            base[tid] = r;
        }
        __syncthreads();
        if (ok) {
            const int32_t r = wcnt[w][ex] + __popcll(below);
            if (capacity > 0 && r - seg[ex] >= capacity) {
                slot[i] = -1;                       // past the expert's capacity
            } else {
                slot[i] = r;
                if (src) src[r] = (int32_t)(i / k);
            }
        } else if (live) {
            slot[i] = -1;
        }
        __syncthreads();
    }
}

static_assert(kMaxExperts == kLayoutScratchExperts, "scratch sized for EP_MAX_EXPERTS");

// ---- one launch for small inputs ----------------------------------------
//
// Up to kLayoutSmallMaxPairs pairs and kSmallMaxExperts experts: a single
// launch of workgroups of 16 wavefronts, each owning a chunk of 1024
// consecutive pairs, one per lane.  There is no second launch and no
// workspace round trip, and no workgroup waits for another: each one
//   1. counts all pairs itself (two per 16-byte load when topk_idx is
//      16-byte aligned; the lines come from L2 after the first fetch), per
//      expert, split into the pairs before its chunk and the rest, and
//      counts its own pairs per (wavefront, expert);
//   2. derives every expert's total and segment start (the same packed,
//      aligned or fixed-stride placement as the two-launch path) and every
//      (wavefront, expert) base row: segment start + the expert's pairs in
//      earlier chunks + those in earlier wavefronts of this chunk;
//   3. ranks its pairs: a pair's rank among the wavefront's pairs of its
//      expert is the popcount of the lower lanes whose expert id matches,
//      found by ballots over the id's bits.
// Atomics produce counts only; no position depends on their order.
// Workgroup 0 writes counts, offsets and the invalid / dropped counts.
// Measured on MI355X against the two launches (rocprofv3 kernel durations,
// caches emptied first): 3.8 against 8.4 us at 256 pairs, 7.2 against
// 9.2 us at 16384 pairs (E 64, k 4); with HIP events the single launch was
// faster up to 16384 pairs for E 8, 64 and 256 and up to 32768 for E 256,
// slower at 32768 for E 64 (13.5 against 12.6 us) and at 65536 (the
// redundant counting grows with the pairs).
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallMaxExperts = 256;

__global__ __launch_bounds__(kSmallThreads)
void layout_single_kernel(const int64_t* __restrict__ idx, int pairs, int k, int E, int alignment,
                          int capacity, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ slot, int32_t* __restrict__ src,
                          int32_t* __restrict__ num_invalid, int32_t* __restrict__ num_dropped)
{
    __shared__ int32_t base[kSmallWaves][kSmallMaxExperts];   // own counts, then base rows
    __shared__ int32_t before[kSmallMaxExperts];
    __shared__ int32_t after[kSmallMaxExperts];
    __shared__ int32_t seg[kSmallMaxExperts];
    __shared__ int32_t waves[kSmallWaves];
    __shared__ int32_t nbad, ndrop;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const bool first = blockIdx.x == 0;
    const int cbeg = blockIdx.x * kSmallThreads;
    const int i = cbeg + tid;               // this lane's own pair

    for (int q = tid; q < kSmallWaves * kSmallMaxExperts; q += kSmallThreads) (&base[0][0])[q] = 0;
    for (int e = tid; e < kSmallMaxExperts; e += kSmallThreads) {
        before[e] = 0;
        after[e] = 0;
    }
    if (tid == 0) {
        nbad = 0;
        ndrop = 0;
    }
    // the own pair's expert id (-1 masked, invalid, or past the end)
    const int64_t e_own = i < pairs ? idx[i] : -1;
    const int32_t ex = (e_own >= 0 && e_own < E) ? (int32_t)e_own : -1;
    __syncthreads();

    // 1. counts: every pair, split at the chunk, and the own pairs per wavefront
    int bad = 0;
    if ((reinterpret_cast<uintptr_t>(idx) & 15u) == 0) {
        const longlong2* v2 = reinterpret_cast<const longlong2*>(idx);
        const int nv = pairs >> 1;
#pragma unroll 8
        for (int v = tid; v < nv; v += kSmallThreads) {
            const longlong2 q = v2[v];
            const int i0 = 2 * v;
            if (q.x >= 0 && q.x < E) atomicAdd(i0 < cbeg ? &before[q.x] : &after[q.x], 1);
            else bad += q.x != -1;
            if (q.y >= 0 && q.y < E) atomicAdd(i0 + 1 < cbeg ? &before[q.y] : &after[q.y], 1);
            else bad += q.y != -1;
        }
        if ((pairs & 1) && tid == 0) {
            const int64_t e = idx[pairs - 1];
            if (e >= 0 && e < E) atomicAdd(pairs - 1 < cbeg ? &before[e] : &after[e], 1);
            else bad += e != -1;
        }
    } else {
#pragma unroll 8
        for (int q = tid; q < pairs; q += kSmallThreads) {
            const int64_t e = idx[q];
            if (e >= 0 && e < E)
                atomicAdd(q < cbeg ? &before[e] : &after[e], 1);
            else
                bad += e != -1;
        }
    }
    if (ex >= 0) atomicAdd(&base[w][ex], 1);
    if (first && bad) atomicAdd(&nbad, bad);
    __syncthreads();

    // 2. totals, segment starts, base rows (thread e < E owns expert e)
    const int32_t tot = tid < E ? before[tid] + after[tid] : 0;
    const int32_t padded = tid < E ? (tot + alignment - 1) / alignment * alignment : 0;
    int32_t n = 0;
    const int32_t run = block_exclusive_scan(padded, waves, &n);
    if (tid < E) {
        const int32_t start = capacity > 0 ? tid * capacity : run;
        seg[tid] = start;
        if (first) {
            counts[tid] = capacity > 0 ? min(tot, capacity) : tot;
            offsets[tid] = start;
            if (capacity > 0 && tot > capacity) atomicAdd(&ndrop, tot - capacity);
        }
        int32_t b = start + before[tid];
        for (int v = 0; v < kSmallWaves; ++v) {
            const int32_t c = base[v][tid];
            base[v][tid] = b;
            b += c;
        }
    }
    if (first && tid == 0) offsets[E] = capacity > 0 ? E * capacity : n;
    __syncthreads();
    if (first && tid == 0) {
        if (num_invalid) *num_invalid = nbad;
        if (num_dropped) *num_dropped = ndrop;
    }

    // 3. ranks within the wavefront
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const bool ok = ex >= 0;
    uint64_t m = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = ok && ((ex >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    if (ok) {
        const int32_t r = base[w][ex] + __popcll(m & ((1ull << lane) - 1ull));
        if (capacity > 0 && r - seg[ex] >= capacity) {
            slot[i] = -1;                           // past the expert's capacity
        } else {
            slot[i] = r;
            if (src) src[r] = i / k;
        }
    } else if (i < pairs) {
        slot[i] = -1;
    }
}

}  // namespace

// Scratch of the no-allocation entry point: room for the largest histogram
// any accepted layout needs (at most kLayoutMaxChunks chunks, a multiple of
// 4, times EP_MAX_EXPERTS experts, plus one invalid-entry count per chunk).
// Each device holds its own copy from the library's load until the process
// ends.  Host code never passes this name to a kernel: on the host it only
// names the symbol, whose device address hipGetSymbolAddress returns.
static __device__ __align__(256) int32_t scratch[kLayoutScratchBytes / sizeof(int32_t)];

static int64_t whole_batches(int64_t n)
{
    return (n + kLayoutThreads - 1) / kLayoutThreads * kLayoutThreads;
}

int64_t layout_chunk_pairs(int64_t pairs)
{
    // a whole number of 256-pair batches; about kLayoutSmallChunks chunks
    // for small inputs, else at least kLayoutMinChunk pairs and at most
    // kLayoutMaxChunks chunks (hidden 2048, k 4: 16384 pairs in 64 chunks of
    // 256 took the layout from 12.9 to about 11 us; at 65536 pairs and
    // beyond the chunks are as before)
    const int64_t small = whole_batches((pairs + kLayoutSmallChunks - 1) / kLayoutSmallChunks);
    const int64_t large = std::max(kLayoutMinChunk,
                                   whole_batches((pairs + kLayoutMaxChunks - 1) / kLayoutMaxChunks));
    return std::max((int64_t)kLayoutThreads, std::min(small, large));
}

int64_t layout_num_chunks(int64_t pairs)
{
    const int64_t chunk = layout_chunk_pairs(pairs);
    return pairs <= 0 ? 1 : (pairs + chunk - 1) / chunk;
}

// chunks padded to a multiple of 4 so each expert's row of the histogram is
// a whole number of 16-byte vectors
static int64_t padded_chunks(int64_t pairs) { return (layout_num_chunks(pairs) + 3) & ~(int64_t)3; }

size_t layout_workspace_bytes(int64_t pairs, int num_experts)
{
    const int64_t Cp = padded_chunks(pairs);
    const size_t bytes = (size_t)(Cp * (int64_t)num_experts + Cp) * sizeof(int32_t);
    return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                         int num_experts, int alignment, int capacity, int32_t* counts,
                         int32_t* offsets, int32_t* slot, int32_t* src, int32_t* num_invalid,
                         int32_t* num_dropped, void* workspace, hipStream_t stream)
{
    const int64_t pairs = num_tokens * (int64_t)num_topk;
    if (pairs <= kLayoutSmallMaxPairs && num_experts <= kSmallMaxExperts) {
        const int groups = (int)((pairs + kSmallThreads - 1) / kSmallThreads);
        hipLaunchKernelGGL(layout_single_kernel, dim3((unsigned)(groups > 0 ? groups : 1)),
                           dim3(kSmallThreads), 0, stream, topk_idx, (int)pairs, num_topk,
                           num_experts, alignment, capacity, counts, offsets, slot, src, num_invalid,
                           num_dropped);
        return hipGetLastError();
    }
    const int64_t chunk = layout_chunk_pairs(pairs);
    const int64_t C = layout_num_chunks(pairs);
    const int64_t Cp = padded_chunks(pairs);
    int32_t* hist = static_cast<int32_t*>(workspace);
    int32_t* bad = hist + Cp * num_experts;

    // Cp workgroups: the padding chunks start past the end and write zeros
    hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)Cp), dim3(kLayoutThreads), 0, stream,
                       topk_idx, pairs, chunk, num_experts, (int)Cp, hist, bad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    if (num_experts <= kWideMaxExperts)
        hipLaunchKernelGGL(layout_scatter_wide_kernel, dim3((unsigned)C), dim3(kWideThreads), 0,
                           stream, topk_idx, pairs, chunk, num_topk, num_experts, (int)Cp, (int)C,
                           alignment, capacity, hist, bad, counts, offsets, slot, src, num_invalid,
                           num_dropped);
    else
        hipLaunchKernelGGL(layout_scatter_kernel, dim3((unsigned)C), dim3(kLayoutThreads), 0, stream,
                           topk_idx, pairs, chunk, num_topk, num_experts, (int)Cp, (int)C,
                           alignment, capacity, hist, bad, counts, offsets, slot, src, num_invalid,
                           num_dropped);
    return hipGetLastError();
}

size_t layout_scratch_bytes() { return sizeof(scratch); }

// Device address of this device's scratch, looked up once per device (with
// that device current) and kept.
hipError_t layout_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace ep

// ep_ranked.hip -- the non-expanded, per-(token, rank) path on gfx950.
//
// Passages: NCCL EP page, nccl_ep.cc: the high-throughput handle's routing
// structures (the all-gathered routing bitmap [tokens, ceil(E/8)], one bit
// per expert; sparse_to_dense_map: the row of a (token, destination rank)
// pair in that rank's buffer, -1 when not routed; local_expert_routing_map
// [max_recv_tokens, experts_per_rank]; num_tokens_for_experts, each token
// counted once per rank), ncclEpCreateHandle's high-throughput branch
// (Step 1 bitmap from topk_idx, Step 2 all-gather, Step 3 preprocessing with
// the per-expert receive counter), and the high-throughput branches of
// ncclEpDispatch / ncclEpCombine (a token row travels once per rank; the
// forward combine carries tokens only).
//
// G ranks; rank d owns experts [d*El, (d+1)*El), El = E / G.  The
// all-gathered map has G*T rows; global token g = s*T + t is token t of
// rank s.  Rank d's receive buffer lists the tokens that select any of its
// experts, once each, in increasing g.
//
// Kernels (all deterministic: atomics only ever OR bits or add counts):
//   routing map:  one workgroup per 64 tokens ORs every slot's bit into an
//                 LDS copy of the rows, then writes the rows out whole.
//   rank count:   one workgroup per chunk of 256 global tokens (more once
//                 there would be over 256 chunks) counts, for every rank,
//                 the chunk's tokens it receives (wavefront ballots over a
//                 per-token rank mask; map rows of up to 8 words stay in
//                 registers, an LDS table gives each expert's rank), and
//                 for the local rank the received tokens per local expert
//                 and the selections past k_out.
//   rank scatter: each workgroup sums the earlier chunks' counts (all its
//                 threads, contiguous loads), then walks its chunk in
//                 batches of 256 tokens; a token's row in rank d's buffer
//                 is that base plus its ballot prefix count in the batch.
//                 It writes sparse_to_dense for the local rank's tokens and
//                 the receive-side rows, and all workgroups clear the rows
//                 past the received count; workgroup 0 also sums the
//                 per-chunk receive-side counts into the totals.
//   dispatch:     one workgroup per (2 KiB tile of a token's row, group of
//                 8 destination ranks), the tile's workgroups back to back
//                 on one XCD; it loads its tile once and stores it, with
//                 streaming stores, to each rank of the group that receives
//                 the token (a table of G row pointers passed by value);
//                 tile 0 also writes the token's weights for those ranks'
//                 experts.  bf16 rows of 257-511 vectors whose last tile
//                 would be at most half full take 64-lane tiles; other rows
//                 under 512 vectors, and 8-bit rows with their scales, take
//                 one workgroup per token that holds the row in registers.  The 8-bit cast sent once per rank is
//                 tiled the same way, each lane casting 16 channels.
//   fused permute: the receiving rank's dispatch with the permute folded
//                 in: one workgroup per received token reads the sender's
//                 row once and stores it to each of the rank's local-expert
//                 rows, with the weights; 8-bit code rows carry their scale
//                 rows along.
//   combine:      one workgroup per (token, 2 KiB tile; 1 KiB where the
//                 last 2 KiB tile would be at most half full) gathers its vectors from the G buffers
//                 through buffer resources (an unrouted rank gets a 0-byte
//                 resource: its loads return 0 without a branch), sums them
//                 in fp32 in increasing rank and stores once, with a
//                 streaming store (rows of at most 64 vectors: one
//                 workgroup per token).

#include <algorithm>

#include "ep_cast.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMaxExperts = 1024;   // EP_MAX_EXPERTS
constexpr int kMapTokens = 64;      // tokens per routing-map workgroup
constexpr int kMapThreads = 256;
constexpr int kMaxRowWords = kMaxExperts / 32;
constexpr int kRankThreads = 256;
constexpr int kRankWaves = kRankThreads / 64;

// ----------------------------------------------------------- routing map

__global__ __launch_bounds__(kMapThreads)
void routing_map_kernel(const int64_t* __restrict__ idx, int64_t T, int k, int E, int W,
                        bool word_rows, uint8_t* __restrict__ map, int32_t* __restrict__ num_invalid)
{
    __shared__ uint32_t rows[kMapTokens * kMaxRowWords];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kMapTokens;
    const int nt = (int)min((int64_t)kMapTokens, T - t0);
    const int W32 = (W + 3) >> 2;
    for (int i = tid; i < nt * W32; i += kMapThreads) rows[i] = 0u;
    __syncthreads();

    int bad = 0;
    const int pairs = nt * k;
    const int64_t* ix = idx + t0 * k;
    for (int i = tid; i < pairs; i += kMapThreads) {
        const int64_t e = ix[i];
        if (e >= 0 && e < E) {
            // bit e of the row: word e / 32, bit e % 32 (little-endian, so
            // byte e / 8 holds it at bit e % 8)
            atomicOr(&rows[(i / k) * W32 + (int)(e >> 5)], 1u << (int)(e & 31));
        } else if (e != -1) {
            ++bad;
        }
    }
    __syncthreads();

    uint8_t* out = map + t0 * W;
    if (word_rows) {
        uint32_t* o32 = reinterpret_cast<uint32_t*>(out);
        for (int i = tid; i < nt * W32; i += kMapThreads) o32[i] = rows[i];
    } else {
        for (int i = tid; i < nt * W; i += kMapThreads) {
            const int tl = i / W;
            const int b = i - tl * W;
            out[i] = (uint8_t)(rows[tl * W32 + (b >> 2)] >> (8 * (b & 3)));
        }
    }
    if (num_invalid != nullptr) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) bad += __shfl_xor(bad, m, 64);
        if ((tid & 63) == 0 && bad != 0) atomicAdd(num_invalid, bad);
    }
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

// ------------------------------------------------------------ rank layout

// One map row.  NW > 0: the row is NW 32-bit words (rows 4-byte aligned)
// held in registers; NW == 0: any width, read from memory byte by byte.
template <int NW>
struct MapRow {
    uint32_t w[NW > 0 ? NW : 1];
    const uint8_t* row;
    int W;

    __device__ __forceinline__ void load(const uint8_t* r, int W_, bool live)
    {
        row = r;
        W = W_;
        if constexpr (NW > 0) {
            const uint32_t* r32 = reinterpret_cast<const uint32_t*>(r);
#pragma unroll
            for (int i = 0; i < NW; ++i) w[i] = live ? r32[i] : 0u;
        }
    }

    __device__ __forceinline__ uint32_t word(int i) const
    {
        uint32_t v = 0u;
#pragma unroll
        for (int j = 0; j < NW; ++j) v = (i == j) ? w[j] : v;
        return v;
    }

    // 32 bits starting at bit p (little-endian bit order), 0 past the row.
    __device__ __forceinline__ uint32_t bits32(int p) const
    {
        if constexpr (NW > 0) {
            const int i = p >> 5;
            const int sh = p & 31;
            const uint32_t lo = word(i);
            const uint32_t hi = word(i + 1);
            return sh == 0 ? lo : ((lo >> sh) | (hi << (32 - sh)));
        } else {
            const int b0 = p >> 3;
            uint64_t v = 0;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int b = b0 + i;
                if (b < W) v |= (uint64_t)row[b] << (8 * i);
            }
            return (uint32_t)(v >> (p & 7));
        }
    }
};

// Bit d of the result: the token selects an expert of rank d.  rank_of is
// the LDS table expert -> rank.
template <int NW>
__device__ __forceinline__ uint64_t rank_mask(const MapRow<NW>& r, int E, const uint8_t* rank_of)
{
    uint64_t m = 0;
    const int nwin = NW > 0 ? NW : (E + 31) / 32;
#pragma unroll
    for (int i = 0; i < (NW > 0 ? NW : 1); ++i) {
        for (int ii = (NW > 0 ? i : 0); ii < (NW > 0 ? i + 1 : nwin); ++ii) {
            const int p = ii * 32;
            uint32_t w = NW > 0 ? r.w[i] : r.bits32(p);
            if (p >= E) w = 0u;
            else if (E - p < 32) w &= (1u << (E - p)) - 1u;
            while (w != 0u) {
                const int e = p + __builtin_ctz(w);
                w &= w - 1u;
                m |= 1ull << rank_of[e];
            }
        }
    }
    return m;
}

__device__ __forceinline__ int popc64(uint64_t v) { return __builtin_popcountll(v); }

__device__ __forceinline__ uint64_t lanes_below()
{
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ void fill_rank_table(uint8_t* rank_of, int E, int El)
{
    for (int e = threadIdx.x; e < E; e += kRankThreads) rank_of[e] = (uint8_t)(e / El);
}

// Workspace (int32, chunk-major so a workgroup's reads are contiguous):
//   cnt[c][d]   tokens of chunk c that rank d receives          (C x G)
//   ecnt[c][e]  of those the local rank receives, how many select local
//               expert e                                          (C x El)
//   ovf[c]      their selections past k_out                      (C)
template <int NW>
__global__ __launch_bounds__(kRankThreads)
void rank_count_kernel(const uint8_t* __restrict__ map, int64_t R, int W, int E, int G, int El,
                       int rank, int k_out, int64_t chunk, int C, int32_t* __restrict__ ws)
{
    __shared__ int32_t s_cnt[kMaxRanks];
    __shared__ int32_t s_ecnt[kMaxExperts];
    __shared__ uint8_t s_rank_of[kMaxExperts];
    __shared__ int32_t s_ovf;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = blockIdx.x;
    const int64_t g0 = (int64_t)c * chunk;
    const int64_t g1 = min(R, g0 + chunk);
    // the first batch's rows are requested before anything else
    MapRow<NW> next;
    if (g0 < g1) next.load(map + min(g0 + tid, g1 - 1) * W, W, g0 + tid < g1);
    if (tid < G) s_cnt[tid] = 0;
    if (tid == 0) s_ovf = 0;
    for (int e = tid; e < El; e += kRankThreads) s_ecnt[e] = 0;
    fill_rank_table(s_rank_of, E, El);
    __syncthreads();

    const int first = rank * El;
    int ovf = 0;
    for (int64_t b = g0; b < g1; b += kRankThreads) {
        const int64_t g = b + tid;
        const bool live = g < g1;
        const MapRow<NW> row = next;
        if (b + kRankThreads < g1)
            next.load(map + min(g + kRankThreads, g1 - 1) * W, W, g + kRankThreads < g1);
        const uint64_t m = live ? rank_mask<NW>(row, E, s_rank_of) : 0ull;
        for (int d = 0; d < G; ++d) {
            const uint64_t bal = __ballot((m >> d) & 1ull);
            if (lane == 0 && bal != 0ull) atomicAdd(&s_cnt[d], popc64(bal));
        }
        if ((m >> rank) & 1ull) {
            int n = 0;
            for (int q = 0; q < El; q += 32) {
                uint32_t wbits = row.bits32(first + q);
                if (El - q < 32) wbits &= (1u << (El - q)) - 1u;
                n += __builtin_popcount(wbits);
                while (wbits != 0u) {
                    const int e = q + __builtin_ctz(wbits);
                    wbits &= wbits - 1u;
                    atomicAdd(&s_ecnt[e], 1);
                }
            }
            ovf += n > k_out ? n - k_out : 0;
        }
    }
    if (ovf != 0) atomicAdd(&s_ovf, ovf);
    __syncthreads();
    int32_t* cnt = ws;
    int32_t* ecnt = ws + (int64_t)C * G;
    int32_t* ovfs = ecnt + (int64_t)C * El;
    if (tid < G) cnt[(int64_t)c * G + tid] = s_cnt[tid];
    for (int e = tid; e < El; e += kRankThreads) ecnt[(int64_t)c * El + e] = s_ecnt[e];
    if (tid == 0) ovfs[c] = s_ovf;
}

// sum of v[cc * stride] over cc = j, j + S, j + 2S, ... below min(C, lim):
// loads are issued eight at a time, so a thread waits about once per eight
// (the tables were written by another kernel, possibly on another XCD).
__device__ __forceinline__ int32_t strided_sum(const int32_t* v, int stride, int j, int S, int C,
                                               int lim)
{
    const int end = min(C, lim);
    int32_t sum = 0;
    for (int cc0 = j; cc0 < end; cc0 += 8 * S) {
        int32_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int cc = cc0 + u * S;
            x[u] = cc < end ? v[(int64_t)cc * stride] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += x[u];
    }
    return sum;
}

// Four local-map bytes (0 or 1) from four bits.
__device__ __forceinline__ uint32_t spread4(uint32_t b)
{
    return (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
}

// Sixteen local-map bytes from the low sixteen bits.
__device__ __forceinline__ uint4 spread16(uint32_t b)
{
    return make_uint4(spread4(b & 15u), spread4((b >> 4) & 15u), spread4((b >> 8) & 15u),
                      spread4((b >> 12) & 15u));
}

// Writes one recv_topk_idx row: the first k_out values put, then -1; with
// `pairs` (k_out even, row 16-byte aligned) two entries per 16-byte store.
struct TopkWriter {
    int64_t* row;
    int k_out;
    bool pairs;
    int n = 0;
    int64_t held = 0;

    __device__ __forceinline__ TopkWriter(int64_t* r, int k, bool p) : row(r), k_out(k), pairs(p) {}

    __device__ __forceinline__ void put(int64_t v)
    {
        if (n < k_out) {
            if (!pairs) {
                row[n] = v;
            } else if (n & 1) {
                *reinterpret_cast<longlong2*>(row + n - 1) = make_longlong2(held, v);
            } else {
                held = v;
            }
        }
        ++n;
    }

    __device__ __forceinline__ void finish()
    {
        while (n < k_out) put(-1);
    }
};

template <int NW>
__global__ __launch_bounds__(kRankThreads)
void rank_scatter_kernel(const uint8_t* __restrict__ map, int64_t R, int64_t T, int W, int E,
                         int G, int El, int rank, int k_out, int64_t chunk, int C,
                         const int32_t* __restrict__ ws, int32_t* __restrict__ s2d,
                         uint8_t* __restrict__ local_map, int32_t* __restrict__ recv_src,
                         int64_t* __restrict__ recv_topk_idx, int32_t* __restrict__ expert_counts,
                         int32_t* __restrict__ num_recv, int32_t* __restrict__ num_overflow)
{
    __shared__ int32_t s_base[kMaxRanks];
    __shared__ int32_t s_wave[kRankWaves][kMaxRanks];
    __shared__ int32_t s_tot[kMaxExperts];
    __shared__ uint8_t s_rank_of[kMaxExperts];
    __shared__ int32_t s_nrecv;
    __shared__ int32_t s_ovf;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = blockIdx.x;
    const int32_t* cnt = ws;
    const int32_t* ecnt = ws + (int64_t)C * G;
    const int32_t* ovfs = ecnt + (int64_t)C * El;
    const int64_t g0 = (int64_t)c * chunk;
    const int64_t g1 = min(R, g0 + chunk);
    // the first batch's rows are requested before the prefix sums
    MapRow<NW> next;
    if (g0 < g1) next.load(map + min(g0 + tid, g1 - 1) * W, W, g0 + tid < g1);
    if (tid < G) s_base[tid] = 0;
    if (tid == 0) {
        s_nrecv = 0;
        s_ovf = 0;
    }
    for (int j = tid; j < kMaxExperts; j += kRankThreads) s_tot[j] = 0;
    fill_rank_table(s_rank_of, E, El);
    __syncthreads();

    // The receive-side totals over all chunks, spread over the workgroups
    // from the last one down (the first ones hold the local rank's tokens
    // and write sparse_to_dense): workgroup C-1-i sums local experts i,
    // i + C, i + 2C, ..., one value per load, eight loads in flight.
    const int ci = C - 1 - c;
    const int my_experts = ci < El ? (El - 1 - ci) / C + 1 : 0;
    {
        const int nv = my_experts * C;
        for (int v0 = tid; v0 < nv; v0 += 8 * kRankThreads) {
            int32_t x[8];
            int j[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = v0 + u * kRankThreads;
                j[u] = v < nv ? v / C : 0;
                x[u] = v < nv ? ecnt[(int64_t)(v - j[u] * C) * El + ci + j[u] * C] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (x[u] != 0) atomicAdd(&s_tot[j[u]], x[u]);
        }
        if (c == 0) {
            const int32_t o = strided_sum(ovfs, 1, tid, kRankThreads, C, C);
            if (o != 0) atomicAdd(&s_ovf, o);
        }
    }

    // Rows of each rank's buffer taken by earlier chunks, and the local
    // rank's received total: thread (d, j) sums column d of chunks j, j + S,
    // j + 2S, ... (S = 256 / G threads per rank, contiguous loads).
    {
        const int S = kRankThreads / G;
        if (tid < S * G) {
            const int d = tid % G;
            const int32_t before = strided_sum(cnt + d, G, tid / G, S, C, c);
            if (before != 0) atomicAdd(&s_base[d], before);
            if (d == rank) {
                const int32_t all = strided_sum(cnt + d, G, tid / G, S, C, C);
                if (all != 0) atomicAdd(&s_nrecv, all);
            }
        }
    }
    __syncthreads();
    if (c == 0 && tid == 0) {
        *num_recv = s_nrecv;
        if (num_overflow != nullptr) *num_overflow = s_ovf;
    }
    for (int j = tid; j < my_experts; j += kRankThreads) expert_counts[ci + j * C] = s_tot[j];

    const bool map4 = (El & 3) == 0;
    // 16-byte stores where rows stay 16-byte aligned
    const bool map16 = (El & 15) == 0 && (reinterpret_cast<uintptr_t>(local_map) & 15u) == 0;
    const bool topk16 = (k_out & 1) == 0 && (reinterpret_cast<uintptr_t>(recv_topk_idx) & 15u) == 0;
    const int first = rank * El;
    const int64_t mine0 = (int64_t)rank * T;
    for (int64_t b = g0; b < g1; b += kRankThreads) {
        const int64_t g = b + tid;
        const bool live = g < g1;
        const MapRow<NW> row = next;
        if (b + kRankThreads < g1)
            next.load(map + min(g + kRankThreads, g1 - 1) * W, W, g + kRankThreads < g1);
        const uint64_t m = live ? rank_mask<NW>(row, E, s_rank_of) : 0ull;
        for (int d = 0; d < G; ++d) {
            const uint64_t bal = __ballot((m >> d) & 1ull);
            if (lane == 0) s_wave[wave][d] = popc64(bal);
        }
        __syncthreads();
        const bool mine = live && g >= mine0 && g < mine0 + T;
        for (int d = 0; d < G; ++d) {
            const bool hit = (m >> d) & 1ull;
            const uint64_t bal = __ballot(hit);
            int32_t pos = s_base[d] + popc64(bal & lanes_below());
            for (int w = 0; w < wave; ++w) pos += s_wave[w][d];
            if (mine) s2d[(g - mine0) * G + d] = hit ? pos : -1;
            if (hit && d == rank) {
                // the receive-side row of token g
                recv_src[pos] = (int32_t)g;
                int64_t* topk = recv_topk_idx + (int64_t)pos * k_out;
                uint8_t* lm = local_map + (int64_t)pos * El;
                TopkWriter tw(topk, k_out, topk16);
                for (int q = 0; q < El; q += 32) {
                    uint32_t wbits = row.bits32(first + q);
                    const int nb = min(32, El - q);
                    if (nb < 32) wbits &= (1u << nb) - 1u;
                    if (map16) {
                        for (int i = 0; i < nb; i += 16)
                            *reinterpret_cast<uint4*>(lm + q + i) = spread16(wbits >> i);
                    } else if (map4) {
                        for (int i = 0; i < nb; i += 4)
                            *reinterpret_cast<uint32_t*>(lm + q + i) = spread4((wbits >> i) & 15u);
                    } else {
                        for (int i = 0; i < nb; ++i) lm[q + i] = (uint8_t)((wbits >> i) & 1u);
                    }
                    while (wbits != 0u) {
                        const int e = q + __builtin_ctz(wbits);
                        wbits &= wbits - 1u;
                        tw.put(e);
                    }
                }
                tw.finish();
            }
        }
        __syncthreads();
        if (tid < G) {
            int32_t sum = 0;
            for (int w = 0; w < kRankWaves; ++w) sum += s_wave[w][tid];
            s_base[tid] += sum;
        }
        __syncthreads();
    }

    // rows past the received count: no source, no local expert
    const int64_t nrecv = s_nrecv;
    const int64_t stride = (int64_t)gridDim.x * kRankThreads;
    for (int64_t i = nrecv + (int64_t)c * kRankThreads + tid; i < R; i += stride) {
        recv_src[i] = -1;
        TopkWriter tw(recv_topk_idx + i * k_out, k_out, topk16);
        tw.finish();
        uint8_t* lm = local_map + i * El;
        if (map16) {
            for (int e = 0; e < El; e += 16) *reinterpret_cast<uint4*>(lm + e) = make_uint4(0u, 0u, 0u, 0u);
        } else if (map4) {
            for (int e = 0; e < El; e += 4) *reinterpret_cast<uint32_t*>(lm + e) = 0u;
        } else {
            for (int e = 0; e < El; ++e) lm[e] = 0;
        }
    }
}

// --------------------------------------------------------------- dispatch

__device__ __forceinline__ void keep(uint4& v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// The token's weights for rank d's experts, written by wavefront 0: lane j
// (< k) holds slot j's expert e_j and weight w_j.  A lane whose expert is
// the first slot of its expert id and belongs to rank d is a "member"; its
// position is the number of members with a smaller expert id, its value the
// fp32 sum in increasing j of the weights of the slots with its id.  Lanes
// j >= members write 0 at position j, so all k positions are written.
__device__ __forceinline__ void write_rank_weights(float* row, int k, int32_t e_j, float sum_j,
                                                   bool first_j, int d, int El)
{
    const int lane = threadIdx.x & 63;
    const bool member = lane < k && first_j && e_j >= d * El && e_j < (d + 1) * El;
    const int members = popc64(__ballot(member));
    int n = 0;
    for (int jj = 0; jj < k; ++jj) {
        const int32_t e2 = __builtin_amdgcn_readlane(e_j, jj);
        const int f2 = __builtin_amdgcn_readlane((int)first_j, jj);
        n += (f2 != 0 && e2 >= d * El && e2 < (d + 1) * El && e2 < e_j) ? 1 : 0;
    }
    if (member) row[n] = sum_j;
    if (lane < k && lane >= members) row[lane] = 0.0f;
}

// Wavefront 0 of a workgroup serving token t: lane j (< k) takes slot j's
// expert and the fp32 sum, in increasing j, of the weights of the slots with
// the same expert, and each rank d in [d0, d1) that receives the token (row
// readlane(p, d) >= 0) gets its weight row.
__device__ __forceinline__ void ranked_token_weights(const int64_t* __restrict__ idx,
                                                     const float* __restrict__ w, int64_t t, int k,
                                                     int E, int El, int32_t p, int d0, int d1,
                                                     const RankPtrs& dw)
{
    const int lane = threadIdx.x & 63;
    const int64_t e64 = lane < k ? idx[t * k + lane] : -1;
    const int32_t e_j = (e64 >= 0 && e64 < E) ? (int32_t)e64 : -1;
    const float w_j = lane < k ? (w ? w[t * k + lane] : 1.0f) : 0.0f;
    float sum = 0.0f;
    bool first = e_j >= 0;
    for (int jj = 0; jj < k; ++jj) {
        const int32_t e2 = __builtin_amdgcn_readlane(e_j, jj);
        const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_j), jj));
        if (e2 == e_j) {
            sum = sum + w2;
            if (jj < lane) first = false;
        }
    }
    for (int d = d0; d < d1; ++d) {
        const int32_t pd = __builtin_amdgcn_readlane(p, d);
        float* base = static_cast<float*>(dw.p[d]);
        if (pd < 0 || base == nullptr) continue;
        write_rank_weights(base + (int64_t)pd * k, k, e_j, sum, first, d, El);
    }
}

// Rows are nvec 16-byte vectors (bf16 tokens, or 8-bit codes); with xs, the
// token's nb fp32 scales are copied to ds[d] as well.  RG == 0: one
// workgroup per token, all G ranks.  RG > 0: one workgroup per (token,
// group of RG ranks), a token's workgroups back to back on one XCD
// (xcd_tile), so its row comes from HBM once.  Used for rows of more than
// 384 vectors when there are more than 4 ranks: for 8-bit rows at hidden
// 7168 (448 vectors) groups of 4 ranks took 75.1 against 83.1 us at 8 ranks
// and 88.6 against 100.2 us at 16 (T=8192 per rank, interleaved A/B;
// groups of 2 were as fast at 8 ranks but 10% slower at 16); for bf16 rows
// of 448 vectors (hidden 3584) 76.4 against 82.9 us and 85.4 against
// 98.1 us (such rows now take 64-lane tiles, below).  At 384 vectors and
// below groups were 2% faster to 41% slower.
template <int NT, int VPT, int RG>
__global__ __launch_bounds__(NT)
void dispatch_ranked_kernel(const uint4* __restrict__ x, int nvec, const int64_t* __restrict__ idx,
                            const float* __restrict__ w, int k, int E, int El, int G,
                            const int32_t* __restrict__ s2d, int64_t dest_rows, RankPtrs dx,
                            RankPtrs dw, bool with_weights, const float* __restrict__ xs,
                            RankPtrs ds, int nb, int64_t num_tokens)
{
    int64_t t = blockIdx.x;
    int gq = 0;
    if (RG > 0 && !xcd_tile(blockIdx.x, (G + RG - 1) / RG, num_tokens, t, gq)) return;
    const int d0 = gq * RG;                        // this workgroup's ranks: d0 .. d1-1
    const int d1 = RG > 0 ? min(G, d0 + RG) : G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // lane d: this token's row in rank d's buffer (-1: not sent; rows past
    // the destination capacity are never written)
    int32_t p = lane < G ? s2d[t * G + lane] : -1;
    if (p >= dest_rows) p = -1;

    if (with_weights && tid < 64) ranked_token_weights(idx, w, t, k, E, El, p, d0, d1, dw);

    if (xs != nullptr) {
        for (int b0 = 0; b0 < nb; b0 += NT) {
            const int b = b0 + tid;
            const float v = b < nb ? xs[t * nb + b] : 0.0f;
            for (int d = d0; d < d1; ++d) {
                const int32_t r = __builtin_amdgcn_readlane(p, d);
                if (r >= 0 && b < nb) static_cast<float*>(ds.p[d])[(int64_t)r * nb + b] = v;
            }
        }
    }

    const uint4* xr = x + t * nvec;
    constexpr int kPass = NT * VPT;
    const int full = nvec / kPass;
    for (int ps = 0; ps < full; ++ps) {
        const int vb = ps * kPass + tid;
        uint4 buf[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) buf[u] = xr[vb + u * NT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) keep(buf[u]);
        for (int d = d0; d < d1; ++d) {
            const int32_t r = __builtin_amdgcn_readlane(p, d);
            if (r < 0) continue;
            const __amdgpu_buffer_rsrc_t dst =
                buffer_rsrc(static_cast<uint4*>(dx.p[d]) + (int64_t)r * nvec, nvec * 16);
#pragma unroll
            for (int u = 0; u < VPT; ++u) store_row16(dst, (vb + u * NT) * 16, buf[u]);
        }
    }
    // ragged tail, the same trip count for every lane (readlane needs the
    // whole wavefront active); past the row end reads 0, stores nothing
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(xr, nvec * 16);
    for (int v0 = full * kPass; v0 < nvec; v0 += NT) {
        const int v = v0 + tid;
        uint4 val = load_row16<0>(xrs, v * 16);
        keep(val);
        for (int d = d0; d < d1; ++d) {
            const int32_t r = __builtin_amdgcn_readlane(p, d);
            if (r >= 0 && v < nvec)
                store_row16(buffer_rsrc(static_cast<uint4*>(dx.p[d]) + (int64_t)r * nvec, nvec * 16),
                            v * 16, val);
        }
    }
}

// Tiled form (no scale rows; token rows of at least 512 vectors, and rows
// of 257-511 vectors whose last 128-lane tile would be at most half full, in
// tiles of NL = 64 lanes): workgroup b maps (XCD-aware) to tile = (token t,
// tile pt of its row) and a group of kRanksPerGroup destination ranks; the
// tile's loads after the first hit the XCD's L2.  Tile 0's workgroups also
// write the group's weight rows.  64-lane tiles against one workgroup per
// token (8 ranks, T=8192 per rank, interleaved A/B): 77.7 against 82.8 us at
// hidden 2560 and 95.5 against 99.8 us at 3584.  8-bit rows with their
// scale rows stay per token: tiled (tile 0 copying the scales) they took
// 99.0 against 98.3 us at hidden 7168 and were 13-35% slower at 8192 and
// 16384.
// The expanded dispatch's tiling, with groups of 8 ranks: a token reaches
// only some of a group's ranks (5.3 of 8 on average with 8 ranks, k=8), so
// a group of 8 stores about as many rows as the expanded dispatch's group
// of 4 slots.  At T=8192, hidden 7168 (interleaved A/B rounds) groups of 8
// took 130.6 against 144.1 us for 4 at 8 ranks and 172.3 against 208.1 us
// at 16 ranks, the same at 4; groups of 2 and 3 were 12-43% slower.
constexpr int kRanksPerGroup = 8;

template <int NL>
__global__ __launch_bounds__(NL)
void dispatch_ranked_tile_kernel(const uint4* __restrict__ x, int nvec,
                                 const int64_t* __restrict__ idx, const float* __restrict__ w,
                                 int k, int E, int El, int G, const int32_t* __restrict__ s2d,
                                 int64_t dest_rows, RankPtrs dx, RankPtrs dw, bool with_weights,
                                 int tpr, int64_t num_tiles, int groups)
{
    int64_t tile;
    int g;
    if (!xcd_tile(blockIdx.x, groups, num_tiles, tile, g)) return;
    const int64_t t = tile / tpr;
    const int pt = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int d0 = g * kRanksPerGroup;
    int32_t p = lane < G ? s2d[t * G + lane] : -1;
    if (p >= dest_rows) p = -1;

    if (with_weights && pt == 0 && tid < 64)
        ranked_token_weights(idx, w, t, k, E, El, p, d0, min(G, d0 + kRanksPerGroup), dw);

    int32_t r[kRanksPerGroup];
#pragma unroll
    for (int q = 0; q < kRanksPerGroup; ++q)
        r[q] = d0 + q < G ? __builtin_amdgcn_readlane(p, d0 + q) : -1;
    const int v = pt * NL + tid;    // past the row end: reads 0, stores nothing
    uint4 val = load_row16<0>(buffer_rsrc(x + t * nvec, nvec * 16), v * 16);
    keep(val);
#pragma unroll
    for (int q = 0; q < kRanksPerGroup; ++q)
        if (r[q] >= 0 && v < nvec)
            store_row16(buffer_rsrc(static_cast<uint4*>(dx.p[d0 + q]) + (int64_t)r[q] * nvec, nvec * 16),
                        v * 16, val);
}

// The 8-bit cast sent once per destination rank: the tiled form above with
// each lane casting one unit of 16 channels (two input vectors, one 16-byte
// code vector; ep_cast.h) instead of copying a vector.  Tiles of NL units
// (64 where the last 128-unit tile would be at most half full, or the row
// has at most 64 units), groups of kRanksPerGroup ranks; the first lane of
// each 8-lane block stores the block's scale (fp32, or the UE8M0 byte) to
// the scale row of each receiving rank.  Units past the row end read zeros
// and store nothing (whole blocks lie on one side of it).
template <int FMT, int SM, int NL>
__global__ __launch_bounds__(NL)
void dispatch_ranked_fp8_tile_kernel(const uint4* __restrict__ x, int nvec,
                                     const int64_t* __restrict__ idx, const float* __restrict__ w,
                                     int k, int E, int El, int G, const int32_t* __restrict__ s2d,
                                     int64_t dest_rows, RankPtrs dq, RankPtrs ds, RankPtrs dw,
                                     bool with_weights, int tpr, int64_t num_tiles, int groups)
{
    int64_t tile;
    int g;
    if (!xcd_tile(blockIdx.x, groups, num_tiles, tile, g)) return;
    const int64_t t = tile / tpr;
    const int pt = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int d0 = g * kRanksPerGroup;
    int32_t p = lane < G ? s2d[t * G + lane] : -1;
    if (p >= dest_rows) p = -1;

    if (with_weights && pt == 0 && tid < 64)
        ranked_token_weights(idx, w, t, k, E, El, p, d0, min(G, d0 + kRanksPerGroup), dw);

    int32_t r[kRanksPerGroup];
#pragma unroll
    for (int q = 0; q < kRanksPerGroup; ++q)
        r[q] = d0 + q < G ? __builtin_amdgcn_readlane(p, d0 + q) : -1;
    const int units = nvec >> 1;
    const int nb = units / kLanesPerBlock;
    const int unit = pt * NL + tid;
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + t * nvec, nvec * 16);
    const uint4 lo = load_row16<0>(xs, unit * 32);
    const uint4 hi = load_row16<0>(xs, unit * 32 + 16);
    uint32_t sb;
    const uint4 code = quantise16<FMT, SM>(lo, hi, sb);
    const int bk = unit / kLanesPerBlock;
    const bool scale_lane = (lane & (kLanesPerBlock - 1)) == 0 && bk < nb;
#pragma unroll
    for (int q = 0; q < kRanksPerGroup; ++q) {
        if (r[q] < 0) continue;
        if (unit < units)
            store_row16(buffer_rsrc(static_cast<uint4*>(dq.p[d0 + q]) + (int64_t)r[q] * units,
                                    units * 16),
                        unit * 16, code);
        if (scale_lane) {
            const int64_t at = (int64_t)r[q] * nb + bk;
            if (SM == kScaleUe8m0)
                static_cast<uint8_t*>(ds.p[d0 + q])[at] = (uint8_t)sb;
            else
                static_cast<uint32_t*>(ds.p[d0 + q])[at] = sb;
        }
    }
}

// ------------------------------------------------ receive side, fused permute

// Received row i: the token (rank s, token t) is read once from rank s's
// rows and stored to each of this rank's local-expert rows slot[i, j];
// wavefront 0 writes the matching weights, the fp32 sum in increasing j' of
// the source weights of the slots that select the pair's expert.  Rows with
// no source return at once.  Tiling a row into 2 KiB pieces (as the send-side
// copies are) took 545 us, or 331 us with one slot group per tile, against
// 307 us for whole rows, at 8 ranks x 8192 tokens, hidden 7168: a received
// row usually has one or two local slots, so most tile workgroups only wait
// on the recv_src -> slot loads and exit.
// SC: the rows are 8-bit codes (nvec 16-byte vectors) and each carries a
// scale row of nb fp32 (src_s[s] [T, nb] -> recv_s [rows, nb]) copied the
// same way.
template <int NT, int VPT, bool SC>
__device__ __forceinline__ void fused_permute_row(
    const RankPtrs& src_x, const RankPtrs& src_s, const RankPtrs& src_idx, const RankPtrs& src_w,
    int64_t T, int nvec, int nb, int k, int E, int El, int G, int rank,
    const int32_t* __restrict__ recv_src, const int64_t* __restrict__ recv_topk_idx,
    const int32_t* __restrict__ slot, int64_t rows, uint4* __restrict__ recv_x,
    float* __restrict__ recv_s, float* __restrict__ recv_w, int64_t i)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the same value in every lane; made scalar so the pointer tables are
    // read with scalar loads
    const int32_t g = __builtin_amdgcn_readfirstlane(recv_src[i]);
    if (g < 0 || g >= (int64_t)G * T) return;   // no source (or not a global token)
    const int s = (int)(g / T);
    const int64_t t = g - (int64_t)s * T;
    int32_t sl = lane < k ? slot[i * k + lane] : -1;
    if (sl >= rows) sl = -1;

    if (recv_w != nullptr && tid < 64) {
        const int64_t le = lane < k ? recv_topk_idx[i * k + lane] : -1;
        const int32_t target = (le >= 0 && le < El) ? rank * El + (int32_t)le : -2;
        const int64_t se = lane < k ? static_cast<const int64_t*>(src_idx.p[s])[t * k + lane] : -1;
        const int32_t se32 = (se >= 0 && se < E) ? (int32_t)se : -3;
        const float* sw = static_cast<const float*>(src_w.p[s]);
        const float swv = lane < k ? (sw ? sw[t * k + lane] : 1.0f) : 0.0f;
        float sum = 0.0f;
        for (int jj = 0; jj < k; ++jj) {
            const int32_t e2 = __builtin_amdgcn_readlane(se32, jj);
            const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swv), jj));
            if (e2 == target) sum = sum + w2;
        }
        if (sl >= 0) recv_w[sl] = sum;
    }

    const uint4* xr = static_cast<const uint4*>(src_x.p[s]) + t * nvec;
    constexpr int kPass = NT * VPT;
    const int full = nvec / kPass;
    for (int ps = 0; ps < full; ++ps) {
        const int vb = ps * kPass + tid;
        uint4 buf[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) buf[u] = xr[vb + u * NT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) keep(buf[u]);
        for (int j = 0; j < k; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(sl, j);
            if (r < 0) continue;
            const __amdgpu_buffer_rsrc_t dst = buffer_rsrc(recv_x + (int64_t)r * nvec, nvec * 16);
#pragma unroll
            for (int u = 0; u < VPT; ++u) store_row16(dst, (vb + u * NT) * 16, buf[u]);
        }
    }
    // ragged tail, the same trip count for every lane (readlane needs the
    // whole wavefront active); past the row end reads 0, stores nothing
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(xr, nvec * 16);
    for (int v0 = full * kPass; v0 < nvec; v0 += NT) {
        const int v = v0 + tid;
        uint4 val = load_row16<0>(xrs, v * 16);
        keep(val);
        for (int j = 0; j < k; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(sl, j);
            if (r >= 0 && v < nvec)
                store_row16(buffer_rsrc(recv_x + (int64_t)r * nvec, nvec * 16), v * 16, val);
        }
    }
    if (SC) {
        // the scale row, one fp32 per lane, the same trip count for every
        // lane
        const float* sr = static_cast<const float*>(src_s.p[s]) + t * nb;
        for (int b0 = 0; b0 < nb; b0 += NT) {
            const int b = b0 + tid;
            const float v = b < nb ? sr[b] : 0.0f;
            for (int j = 0; j < k; ++j) {
                const int32_t r = __builtin_amdgcn_readlane(sl, j);
                if (r >= 0 && b < nb) recv_s[(int64_t)r * nb + b] = v;
            }
        }
    }
}

// Only the first n rows are visited, n the received count read on the
// device (all G*T rows when num_recv is NULL): no host round trip, and the
// rows past it cost one scalar load each.  One workgroup per row (the grid
// is capped at kFusedPermuteGrid, workgroup b taking rows b, b + gridDim.x,
// ... past it).  At 8 ranks x 8192 tokens, hidden 7168, rank 0: 306 us,
// the same as before the bound (the rows past the count exited at once
// anyway); persistent grids of 2048-16384 workgroups took 315-322 us;
// non-temporal or sc1 loads of the source rows, and issuing the row loads
// before the weights, 302-309 us.  The kernel moves a 40/60 mix of reads
// and writes at the rate of a device-to-device copy.
constexpr int64_t kFusedPermuteGrid = 1 << 30;
template <int NT, int VPT, bool SC>
__global__ __launch_bounds__(NT)
void dispatch_fused_permute_kernel(RankPtrs src_x, RankPtrs src_s, RankPtrs src_idx, RankPtrs src_w,
                                   int64_t T, int nvec, int nb, int k, int E, int El, int G,
                                   int rank, const int32_t* __restrict__ recv_src,
                                   const int64_t* __restrict__ recv_topk_idx,
                                   const int32_t* __restrict__ num_recv,
                                   const int32_t* __restrict__ slot, int64_t rows,
                                   uint4* __restrict__ recv_x, float* __restrict__ recv_s,
                                   float* __restrict__ recv_w)
{
    const int64_t R = (int64_t)G * T;
    int64_t n = R;
    if (num_recv != nullptr) {
        const int64_t c = __builtin_amdgcn_readfirstlane(*num_recv);
        n = c < 0 ? 0 : (c < R ? c : R);
    }
    for (int64_t i = blockIdx.x; i < n; i += gridDim.x)
        fused_permute_row<NT, VPT, SC>(src_x, src_s, src_idx, src_w, T, nvec, nb, k, E, El, G,
                                       rank, recv_src, recv_topk_idx, slot, rows, recv_x, recv_s,
                                       recv_w, i);
}

// ---------------------------------------------------------------- combine


__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void add8(float (&acc)[8], const uint4& v)
{
    acc[0] += bf16_lo(v.x);
    acc[1] += bf16_hi(v.x);
    acc[2] += bf16_lo(v.y);
    acc[3] += bf16_hi(v.y);
    acc[4] += bf16_lo(v.z);
    acc[5] += bf16_hi(v.z);
    acc[6] += bf16_lo(v.w);
    acc[7] += bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&acc)[8])
{
    uint4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    return o;
}

// Resource over one source row (0 bytes when the rank holds no row of the
// token: its loads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t src_rsrc(const void* base, int32_t r, int nvec)
{
    const uint4* row = static_cast<const uint4*>(base) + (int64_t)(r < 0 ? 0 : r) * nvec;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(row), (short)0, r < 0 ? 0 : nvec * 16,
                                             0x00020000);
}

__device__ __forceinline__ uint4 load16_nt(__amdgpu_buffer_rsrc_t rs, int v)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, v * 16, 0, 2));
}

// Ranks in groups of 8 (loads of a group back to back), U column vectors
// per lane per iteration.  Adding a 0 from an absent rank leaves the sum
// unchanged: it starts at +0, so it is never -0.
template <int NT, int U>
__global__ __launch_bounds__(NT)
void combine_ranked_kernel(RankPtrs src, int64_t src_rows, const int32_t* __restrict__ s2d, int nvec,
                           int G, uint4* __restrict__ out)
{
    constexpr int kGroup = 8;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    int32_t p = lane < G ? s2d[t * G + lane] : -1;
    if (p >= src_rows) p = -1;
    const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(out + t * nvec, nvec * 16);
    // the same trip count for every lane (readlane needs the whole wavefront
    // active); vectors past the row end read 0 and are not stored
    for (int vb = 0; vb < nvec; vb += NT * U) {
        const int v0 = vb + tid;
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
        for (int d0 = 0; d0 < G; d0 += kGroup) {
            __amdgpu_buffer_rsrc_t rs[kGroup];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const int d = d0 + j;
                const int32_t r = d < G ? __builtin_amdgcn_readlane(p, d) : -1;
                rs[j] = src_rsrc(d < G ? src.p[d] : src.p[0], r, nvec);
            }
            uint4 val[U][kGroup];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < kGroup; ++j) val[u][j] = load16_nt(rs[j], v0 + u * NT);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < kGroup; ++j) add8(acc[u], val[u][j]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (v0 + u * NT < nvec) store_row16(ors, (v0 + u * NT) * 16, pack8(acc[u]));
    }
}

// Tiled form (rows of more than 64 vectors): workgroup b is tile b % tpr of
// token b / tpr, NL vectors, one 16-byte column vector per lane, stored once
// with a streaming store (the expanded combine's tiling; its measurements
// apply).  NL is 128, or 64 where the last 128-lane tile would be at most
// half full (narrow_tiles): at 8 ranks x 8192 tokens those took 24.2, 26.6,
// 30.7 and 64.4 us at hidden 1152, 1280, 1536 and 3584 against 27.4, 28.2,
// 31.6 and 66.6 us in 128-lane tiles.
template <int NL>
__global__ __launch_bounds__(NL)
void combine_ranked_tile_kernel(RankPtrs src, int64_t src_rows, const int32_t* __restrict__ s2d,
                                int nvec, int G, int tpr, uint4* __restrict__ out)
{
    constexpr int kGroup = 8;
    const int64_t tile = blockIdx.x;
    const int64_t t = tile / tpr;
    const int pt = (int)(tile - t * tpr);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    int32_t p = lane < G ? s2d[t * G + lane] : -1;
    if (p >= src_rows) p = -1;
    const int v = pt * NL + tid;            // past the row end: reads 0, stores nothing
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int d0 = 0; d0 < G; d0 += kGroup) {
        uint4 val[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            const int d = d0 + j;
            const int32_t r = d < G ? __builtin_amdgcn_readlane(p, d) : -1;
            val[j] = load16_nt(src_rsrc(d < G ? src.p[d] : src.p[0], r, nvec), v);
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) add8(acc, val[j]);
    }
    if (v < nvec) store_row16(buffer_rsrc(out + t * nvec, nvec * 16), v * 16, pack8(acc));
}

}  // namespace

// ------------------------------------------------------------- launchers

hipError_t launch_routing_map(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                              int num_experts, uint8_t* map, int32_t* num_invalid,
                              hipStream_t stream)
{
    if (num_invalid != nullptr) {
        hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, stream, num_invalid);
        if (num_tokens == 0) return hipGetLastError();
    }
    if (num_tokens == 0) return hipSuccess;
    const int W = (num_experts + 7) / 8;
    const bool words = (W & 3) == 0 && (reinterpret_cast<uintptr_t>(map) & 3u) == 0;
    const dim3 grid((unsigned)((num_tokens + kMapTokens - 1) / kMapTokens));
    hipLaunchKernelGGL(routing_map_kernel, grid, dim3(kMapThreads), 0, stream, topk_idx,
                       num_tokens, num_topk, num_experts, W, words, map, num_invalid);
    return hipGetLastError();
}

// Chunks of global tokens for the rank layout: 256 tokens (one batch), or
// more once there would be over 256 chunks.
static int64_t rank_chunk(int64_t R)
{
    const int64_t need = (R + 255) / 256;
    const int64_t c = (need + kRankThreads - 1) / kRankThreads * kRankThreads;
    return c < kRankThreads ? kRankThreads : c;
}

static int rank_chunks(int64_t R) { return R <= 0 ? 1 : (int)((R + rank_chunk(R) - 1) / rank_chunk(R)); }

size_t rank_layout_workspace_bytes(int64_t tokens_per_rank, int num_experts, int num_ranks)
{
    const int64_t C = rank_chunks(tokens_per_rank * num_ranks);
    return (size_t)(C * (num_ranks + num_experts / num_ranks + 1)) * sizeof(int32_t);
}

template <int NW>
static void launch_rank_shape(hipStream_t stream, const uint8_t* map, int64_t R, int64_t T, int W,
                              int E, int G, int El, int rank, int k_out, int64_t chunk, int C,
                              int32_t* cnt, int32_t* s2d, uint8_t* local_map, int32_t* recv_src,
                              int64_t* recv_topk_idx, int32_t* expert_counts, int32_t* num_recv,
                              int32_t* num_overflow)
{
    hipLaunchKernelGGL(rank_count_kernel<NW>, dim3(C), dim3(kRankThreads), 0, stream, map, R, W, E,
                       G, El, rank, k_out, chunk, C, cnt);
    hipLaunchKernelGGL(rank_scatter_kernel<NW>, dim3(C), dim3(kRankThreads), 0, stream, map, R, T,
                       W, E, G, El, rank, k_out, chunk, C, cnt, s2d, local_map, recv_src,
                       recv_topk_idx, expert_counts, num_recv, num_overflow);
}

hipError_t launch_rank_layout(const uint8_t* map, int64_t tokens_per_rank, int num_experts,
                              int num_ranks, int rank, int k_out, int32_t* s2d,
                              uint8_t* local_map, int32_t* recv_src, int64_t* recv_topk_idx,
                              int32_t* expert_counts, int32_t* num_recv, int32_t* num_overflow,
                              void* workspace, hipStream_t stream)
{
    const int64_t T = tokens_per_rank;
    const int G = num_ranks;
    const int E = num_experts;
    const int El = E / G;
    const int W = (E + 7) / 8;
    const int64_t R = T * G;
    // an empty map still clears and writes the totals (one workgroup each)
    const int64_t chunk = rank_chunk(R);
    const int C = rank_chunks(R);
    int32_t* cnt = static_cast<int32_t*>(workspace);
    // rows of up to 8 aligned words are held in registers
    const bool words = (W & 3) == 0 && (reinterpret_cast<uintptr_t>(map) & 3u) == 0;
    const int nw = words && W / 4 <= 8 ? W / 4 : 0;
#define EP_RL(NW)                                                                               \
    launch_rank_shape<NW>(stream, map, R, T, W, E, G, El, rank, k_out, chunk, C, cnt, s2d,      \
                          local_map, recv_src, recv_topk_idx, expert_counts, num_recv,          \
                          num_overflow)
    switch (nw) {
    case 1: EP_RL(1); break;
    case 2: EP_RL(2); break;
    case 3: EP_RL(3); break;
    case 4: EP_RL(4); break;
    case 5: EP_RL(5); break;
    case 6: EP_RL(6); break;
    case 7: EP_RL(7); break;
    case 8: EP_RL(8); break;
    default: EP_RL(0); break;
    }
#undef EP_RL
    return hipGetLastError();
}

constexpr int kRankGroup = 4;            // ranks per workgroup when grouped
constexpr int kRankGroupVectors = 384;   // grouped for rows of more than this many vectors

hipError_t launch_dispatch_ranked(const void* x, const int64_t* topk_idx, const float* topk_weights,
                                  int64_t num_tokens, int row_bytes, int num_topk, int num_experts,
                                  int num_ranks, const int32_t* s2d, const RankPtrs& dest_x,
                                  const RankPtrs& dest_w, bool with_weights, const float* x_scales,
                                  const RankPtrs& dest_scales, int num_scales, int64_t dest_rows,
                                  hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = row_bytes / 16;
    const dim3 grid((unsigned)num_tokens);
    const uint4* xx = static_cast<const uint4*>(x);
    const int El = num_experts / num_ranks;
    const bool narrow = nvec > 2 * kTileLanes && nvec < kMinTiledDispatchVectors && narrow_tiles(nvec);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (nvec + lanes - 1) / lanes;
    const int groups = (num_ranks + kRanksPerGroup - 1) / kRanksPerGroup;
    const int64_t num_tiles = num_tokens * tpr;
    const int64_t blocks = (num_tiles + 7) / 8 * 8 * groups;
    if (x_scales == nullptr && (narrow || nvec >= kMinTiledDispatchVectors) && blocks <= INT32_MAX) {
#define EP_RT(NL)                                                                               \
    hipLaunchKernelGGL((dispatch_ranked_tile_kernel<NL>), dim3((unsigned)blocks), dim3(NL), 0,      \
                       stream, xx, nvec, topk_idx, topk_weights, num_topk, num_experts, El,        \
                       num_ranks, s2d, dest_rows, dest_x, dest_w, with_weights, tpr, num_tiles,    \
                       groups)
        if (narrow)
            EP_RT(kTileLanes / 2);
        else
            EP_RT(kTileLanes);
#undef EP_RT
        return hipGetLastError();
    }
    // rows of more than kRankGroupVectors vectors: one workgroup per
    // (token, group of kRankGroup ranks)
    const int rgroups = (num_ranks + kRankGroup - 1) / kRankGroup;
    const int64_t gblocks = (num_tokens + 7) / 8 * 8 * rgroups;
    const bool rank_grouped = nvec > kRankGroupVectors && num_ranks > kRankGroup &&
                              gblocks <= INT32_MAX;
    const dim3 ggrid((unsigned)gblocks);
#define EP_DR(NT, V)                                                                            \
    if (rank_grouped)                                                                           \
        hipLaunchKernelGGL((dispatch_ranked_kernel<NT, V, kRankGroup>), ggrid, dim3(NT),          \
                           0, stream, xx, nvec, topk_idx, topk_weights, num_topk, num_experts, El, \
                           num_ranks, s2d, dest_rows, dest_x, dest_w, with_weights, x_scales,      \
                           dest_scales, num_scales, num_tokens);                                  \
    else                                                                                        \
        hipLaunchKernelGGL((dispatch_ranked_kernel<NT, V, 0>), grid, dim3(NT), 0, stream, xx,     \
                           nvec, topk_idx, topk_weights, num_topk, num_experts, El, num_ranks,     \
                           s2d, dest_rows, dest_x, dest_w, with_weights, x_scales, dest_scales,    \
                           num_scales, num_tokens)
    if (nvec <= 64) {
        EP_DR(64, 1);
        return hipGetLastError();
    }
    // 64 lanes when the row is whole 64-lane passes of at most 8 vectors
    // and not whole 128-lane passes (448 = 64 * 7: 8-bit codes at 7168)
    if (nvec % 128 != 0 && nvec % 64 == 0 && nvec <= 64 * 8) {
        switch (nvec / 64) {
        case 2: EP_DR(64, 2); break;
        case 3: EP_DR(64, 3); break;
        case 4: EP_DR(64, 4); break;
        case 5: EP_DR(64, 5); break;
        case 6: EP_DR(64, 6); break;
        case 7: EP_DR(64, 7); break;
        default: EP_DR(64, 8); break;
        }
        return hipGetLastError();
    }
    // 128 lanes with the largest VPT <= 8 whose pass divides the row
    // (896 = 128 * 7 at hidden 7168), else the widest that fits
    const int fit = nvec / 128;
    int vpt = fit < 1 ? 1 : (fit > 8 ? 8 : fit);
    for (int v = 8; v >= 1; --v) {
        if (nvec % (128 * v) == 0) {
            vpt = v;
            break;
        }
    }
    switch (vpt) {
    case 1: EP_DR(128, 1); break;
    case 2: EP_DR(128, 2); break;
    case 3: EP_DR(128, 3); break;
    case 4: EP_DR(128, 4); break;
    case 5: EP_DR(128, 5); break;
    case 6: EP_DR(128, 6); break;
    case 7: EP_DR(128, 7); break;
    default: EP_DR(128, 8); break;
    }
#undef EP_DR
    return hipGetLastError();
}

static int ranked_fp8_lanes(int units)
{
    return units <= 64 || narrow_tiles(units) ? kTileLanes / 2 : kTileLanes;
}

int64_t ranked_fp8_blocks(int64_t num_tokens, int hidden, int num_ranks)
{
    const int units = hidden / 16;
    const int lanes = ranked_fp8_lanes(units);
    const int64_t num_tiles = num_tokens * ((units + lanes - 1) / lanes);
    const int groups = (num_ranks + kRanksPerGroup - 1) / kRanksPerGroup;
    return (num_tiles + 7) / 8 * 8 * groups;
}

hipError_t launch_dispatch_ranked_fp8(const void* x, const int64_t* topk_idx,
                                      const float* topk_weights, int64_t num_tokens, int hidden,
                                      int num_topk, int num_experts, int num_ranks,
                                      const int32_t* s2d, int format, int scale_mode,
                                      const RankPtrs& dest_q, const RankPtrs& dest_scales,
                                      const RankPtrs& dest_w, bool with_weights, int64_t dest_rows,
                                      hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const int units = hidden / 16;
    const int lanes = ranked_fp8_lanes(units);
    const int tpr = (units + lanes - 1) / lanes;
    const int groups = (num_ranks + kRanksPerGroup - 1) / kRanksPerGroup;
    const int64_t num_tiles = num_tokens * tpr;
    const int64_t blocks = ranked_fp8_blocks(num_tokens, hidden, num_ranks);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const int El = num_experts / num_ranks;
    const uint4* xx = static_cast<const uint4*>(x);
#define EP_RF8(F, M, NL)                                                                        \
    hipLaunchKernelGGL((dispatch_ranked_fp8_tile_kernel<F, M, NL>), dim3((unsigned)blocks),       \
                       dim3(NL), 0, stream, xx, nvec, topk_idx, topk_weights, num_topk,            \
                       num_experts, El, num_ranks, s2d, dest_rows, dest_q, dest_scales, dest_w,    \
                       with_weights, tpr, num_tiles, groups)
#define EP_RF8_MODE(F, M)                                                                       \
    if (lanes == kTileLanes) EP_RF8(F, M, kTileLanes); else EP_RF8(F, M, kTileLanes / 2)
    if (format == kE5M2) {
        if (scale_mode == kScalePow2) EP_RF8_MODE(kE5M2, kScalePow2);
        else if (scale_mode == kScaleUe8m0) EP_RF8_MODE(kE5M2, kScaleUe8m0);
        else EP_RF8_MODE(kE5M2, kScaleFp32);
    } else {
        if (scale_mode == kScalePow2) EP_RF8_MODE(kE4M3, kScalePow2);
        else if (scale_mode == kScaleUe8m0) EP_RF8_MODE(kE4M3, kScaleUe8m0);
        else EP_RF8_MODE(kE4M3, kScaleFp32);
    }
#undef EP_RF8_MODE
#undef EP_RF8
    return hipGetLastError();
}

static hipError_t launch_fused_permute_rows(const RankPtrs& src_x, const RankPtrs& src_s,
                                            const RankPtrs& src_idx, const RankPtrs& src_w,
                                            int64_t tokens_per_rank, int nvec, int nb,
                                            int num_topk, int num_experts, int num_ranks,
                                            int rank, const int32_t* recv_src,
                                            const int64_t* recv_topk_idx, const int32_t* num_recv,
                                            const int32_t* slot, int64_t rows, void* recv_x,
                                            float* recv_s, float* recv_w, hipStream_t stream)
{
    const int64_t R = tokens_per_rank * num_ranks;
    if (R == 0) return hipSuccess;
    const dim3 grid((unsigned)std::min(R, kFusedPermuteGrid));
    const int El = num_experts / num_ranks;
    uint4* rx = static_cast<uint4*>(recv_x);
    const bool sc = recv_s != nullptr;
#define EP_FP_SC(NT, V, SC)                                                                      \
    hipLaunchKernelGGL((dispatch_fused_permute_kernel<NT, V, SC>), grid, dim3(NT), 0, stream,      \
                       src_x, src_s, src_idx, src_w, tokens_per_rank, nvec, nb, num_topk,          \
                       num_experts, El, num_ranks, rank, recv_src, recv_topk_idx, num_recv, slot,  \
                       rows, rx, recv_s, recv_w)
#define EP_FP(NT, V)                                                                            \
    if (sc) { EP_FP_SC(NT, V, true); } else { EP_FP_SC(NT, V, false); }
    if (nvec <= 64) {
        EP_FP(64, 1);
        return hipGetLastError();
    }
    // whole passes of 128 lanes if some vpt <= 8 gives them, else whole
    // passes of 64 lanes (an 8-bit row of 7168 bytes: 448 vectors, 64 x 7),
    // else 128 lanes and a ragged tail
    const int fit = nvec / 128;
    int vpt = fit < 1 ? 1 : (fit > 8 ? 8 : fit);
    int nt = 0;
    for (int v = 8; v >= 1 && !nt; --v)
        if (nvec % (128 * v) == 0) nt = 128, vpt = v;
    for (int v = 8; v >= 1 && !nt; --v)
        if (nvec % (64 * v) == 0) nt = 64, vpt = v;
    if (nt == 64) {
        switch (vpt) {
        case 1: EP_FP(64, 1); break;
        case 2: EP_FP(64, 2); break;
        case 3: EP_FP(64, 3); break;
        case 4: EP_FP(64, 4); break;
        case 5: EP_FP(64, 5); break;
        case 6: EP_FP(64, 6); break;
        case 7: EP_FP(64, 7); break;
        default: EP_FP(64, 8); break;
        }
        return hipGetLastError();
    }
    switch (vpt) {
    case 1: EP_FP(128, 1); break;
    case 2: EP_FP(128, 2); break;
    case 3: EP_FP(128, 3); break;
    case 4: EP_FP(128, 4); break;
    case 5: EP_FP(128, 5); break;
    case 6: EP_FP(128, 6); break;
    case 7: EP_FP(128, 7); break;
    default: EP_FP(128, 8); break;
    }
#undef EP_FP
#undef EP_FP_SC
    return hipGetLastError();
}

hipError_t launch_dispatch_fused_permute(const RankPtrs& src_x, const RankPtrs& src_idx,
                                         const RankPtrs& src_w, int64_t tokens_per_rank,
                                         int hidden, int num_topk, int num_experts, int num_ranks,
                                         int rank, const int32_t* recv_src,
                                         const int64_t* recv_topk_idx, const int32_t* num_recv,
                                         const int32_t* slot, int64_t rows, void* recv_x,
                                         float* recv_w, hipStream_t stream)
{
    const RankPtrs none = {};
    return launch_fused_permute_rows(src_x, none, src_idx, src_w, tokens_per_rank, hidden / 8, 0,
                                     num_topk, num_experts, num_ranks, rank, recv_src,
                                     recv_topk_idx, num_recv, slot, rows, recv_x, nullptr, recv_w,
                                     stream);
}

hipError_t launch_dispatch_fused_permute_prequant(const RankPtrs& src_q, const RankPtrs& src_s,
                                                  const RankPtrs& src_idx, const RankPtrs& src_w,
                                                  int64_t tokens_per_rank, int hidden,
                                                  int num_topk, int num_experts, int num_ranks,
                                                  int rank, const int32_t* recv_src,
                                                  const int64_t* recv_topk_idx,
                                                  const int32_t* num_recv, const int32_t* slot,
                                                  int64_t rows, void* recv_q, float* recv_s,
                                                  float* recv_w, hipStream_t stream)
{
    return launch_fused_permute_rows(src_q, src_s, src_idx, src_w, tokens_per_rank, hidden / 16,
                                     hidden / 128, num_topk, num_experts, num_ranks, rank, recv_src,
                                     recv_topk_idx, num_recv, slot, rows, recv_q, recv_s, recv_w,
                                     stream);
}


hipError_t launch_combine_ranked(const RankPtrs& src_y, int64_t src_rows, const int32_t* s2d,
                                 int64_t num_tokens, int hidden, int num_ranks, void* out,
                                 hipStream_t stream)
{
    if (num_tokens == 0) return hipSuccess;
    const int nvec = hidden / 8;
    const dim3 grid((unsigned)num_tokens);
    uint4* oo = static_cast<uint4*>(out);
    const bool narrow = narrow_tiles(nvec);
    const int lanes = narrow ? kTileLanes / 2 : kTileLanes;
    const int tpr = (nvec + lanes - 1) / lanes;
    const int64_t tiles = num_tokens * tpr;
    if (nvec > 64 && tiles <= INT32_MAX) {
        if (narrow)
            hipLaunchKernelGGL(combine_ranked_tile_kernel<kTileLanes / 2>, dim3((unsigned)tiles),
                               dim3(kTileLanes / 2), 0, stream, src_y, src_rows, s2d, nvec,
                               num_ranks, tpr, oo);
        else
            hipLaunchKernelGGL(combine_ranked_tile_kernel<kTileLanes>, dim3((unsigned)tiles),
                               dim3(kTileLanes), 0, stream, src_y, src_rows, s2d, nvec, num_ranks,
                               tpr, oo);
        return hipGetLastError();
    }
    if (nvec <= 64)
        hipLaunchKernelGGL((combine_ranked_kernel<64, 1>), grid, dim3(64), 0, stream, src_y,
                           src_rows, s2d, nvec, num_ranks, oo);
    else if (nvec < 512)
        hipLaunchKernelGGL((combine_ranked_kernel<128, 2>), grid, dim3(128), 0, stream, src_y,
                           src_rows, s2d, nvec, num_ranks, oo);
    else
        hipLaunchKernelGGL((combine_ranked_kernel<256, 2>), grid, dim3(256), 0, stream, src_y,
                           src_rows, s2d, nvec, num_ranks, oo);
    return hipGetLastError();
}

// ---- backward of the once-per-rank dispatch: the weight gradients
//
// NCCL EP page, ncclEpCombine high-throughput branch (the backward combine
// returns the top-k weight gradients: each receiver's [rows, k] gradients,
// aligned with its recv_topk_idx, made dense over its local experts, then
// brought back to [T, k] through the sender's routing rows).  Both steps are
// fused on the sender's side: one lane per (token, slot) with expert e of
// rank d = e / El reads receiver d's row sparse_to_dense[t, d] at position
// n = the number of distinct experts of rank d the token selects below e,
// which is where that receiver lists e.  Masked or invalid slots, and rows
// outside [0, src_rows), get 0.
__global__ __launch_bounds__(256)
void ranked_weight_grad_kernel(RankPtrs grad_w, int64_t src_rows, const int64_t* __restrict__ idx,
                               const int32_t* __restrict__ s2d, int64_t pairs, int k, int E,
                               int G, float* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= pairs) return;
    const int64_t t = i / k;
    const int64_t e = idx[i];
    float g = 0.0f;
    if (e >= 0 && e < E) {
        const int El = E / G;
        const int d = (int)(e / El);
        const int32_t row = s2d[t * G + d];
        const float* src = static_cast<const float*>(grad_w.p[d]);
        if (row >= 0 && row < src_rows && src != nullptr) {
            const int64_t* ti = idx + t * k;
            int n = 0;
            for (int j = 0; j < k; ++j) {
                const int64_t ej = ti[j];
                if (ej < (int64_t)d * El || ej >= e) continue;
                bool first = true;   // count each selected expert once
                for (int q = 0; q < j; ++q) first = first && ti[q] != ej;
                n += first;
            }
            g = src[(int64_t)row * k + n];
        }
    }
    out[i] = g;
}

hipError_t launch_ranked_weight_grad(const RankPtrs& grad_w, int64_t src_rows,
                                     const int64_t* topk_idx, const int32_t* s2d,
                                     int64_t num_tokens, int num_topk, int num_experts,
                                     int num_ranks, float* grad_topk_weights, hipStream_t stream)
{
    const int64_t pairs = num_tokens * num_topk;
    if (pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(ranked_weight_grad_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                       stream, grad_w, src_rows, topk_idx, s2d, pairs, num_topk, num_experts,
                       num_ranks, grad_topk_weights);
    return hipGetLastError();
}

}  // namespace ep

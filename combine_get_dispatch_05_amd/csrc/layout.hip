// layout.hip -- routing layout on gfx950: counts, membership, prefix matrices
// and index maps of one GPU's tokens.
//
// Computes the quantities of "DeepEP Buffer Class API for Expert Parallel
// Communication" (section "Configuration and Layout Helpers":
// num_tokens_per_rank, is_token_in_rank, and the per-expert counts) and the
// handle matrices of "How DeepEP Optimizes Handle Reuse for Repeated
// Dispatches" (section "What the Handle Contains": rank_prefix_matrix,
// channel_prefix_matrix, recv_channel_prefix_matrix, recv_src_idx,
// is_token_in_rank, send_head).
//
// Two launches, stream-ordered (three for more than 16K tokens):
//   count: each lane builds its token's rank bitmask; one ballot per rank
//          gives a 64-token wave's membership mask for that rank, whose
//          popcount is the wave's count; 512-token blocks turn those into
//          within-block offsets in LDS and publish per-rank block totals.
//          Expert counts go to an LDS-privatised histogram per block.
//   (scan: for many blocks, one block turns the block totals into bases.)
//   pos:   one 64-token tile per block.  It sums the block totals it needs
//          (one batch of independent loads), so no block ever waits for
//          another; every (token, rank) cell's position is a tile base plus
//          a popcount, computed flat across the block so that [T][R] rows
//          (send_head, is_token_in_rank) are written by contiguous lanes; one
//          wave then emits each token's destination rows in ascending rank
//          order, the list the pack and reduce kernels read.  Block 0 writes
//          the totals (counts, rank_prefix_matrix, channel entries at the
//          last token).
// Positions come from ballots and scans, never from atomics, so every output
// is deterministic and segments are in token order.
//
// An optional rank mask ("Dynamic Rank Masking" of the same page: nonzero =
// masked) is folded in where membership is formed: every block ANDs the
// tokens' rank bitmasks with the live ranks, and the expert histogram skips
// slots on masked ranks, so a masked rank's slots act as masked slots.

#include <atomic>

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kCountBlock = 512;  // 8 wavefronts = 512 tokens per count block

// Live ranks as NW 64-bit words in LDS (bit r: rank r exists and is not
// masked), one ballot per word.  The caller synchronizes before reading.
template <int NW>
__device__ __forceinline__ void build_live(const int32_t *__restrict__ rank_mask, int R,
                                           uint64_t *s_live)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    for (int w = threadIdx.x / kWave; w < NW; w += nwaves) {
        const int r = w * kWave + lane;
        const bool live = r < R && (rank_mask == nullptr || rank_mask[r] == 0);
        const uint64_t b = wave_ballot(live);
        if (lane == 0)
            s_live[w] = b;
    }
}

// Rank of expert e: a shift when E/R is a power of two (epr_shift >= 0),
// else a division.
__device__ __forceinline__ int rank_of(int e, int epr, int epr_shift)
{
    return epr_shift >= 0 ? e >> epr_shift : e / epr;
}

constexpr int kIdChunk = 8;  // top-k ids loaded per batch (all loads in flight at once)

// Slots k0 .. k0+kIdChunk-1 of a token's row (-1 past K).
__device__ __forceinline__ void load_ids(const int64_t *__restrict__ row, int k0, int K,
                                         int64_t (&ids)[kIdChunk])
{
#pragma unroll
    for (int q = 0; q < kIdChunk; ++q)
        ids[q] = k0 + q < K ? row[k0 + q] : -1;
}

template <int NW>
__device__ __forceinline__ void add_ranks(const int64_t (&ids)[kIdChunk], int E, int epr,
                                          int epr_shift, uint64_t (&m)[NW])
{
#pragma unroll
    for (int q = 0; q < kIdChunk; ++q) {
        const int64_t e = ids[q];
        if (e >= 0 && e < E) {
            const int r = rank_of(int(e), epr, epr_shift);
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if ((r >> 6) == w)
                    m[w] |= 1ull << (r & 63);
        }
    }
}

// Rank bitmask of one token's valid slots (before masking ranks).  The first
// kIdChunk ids are returned in ids0 for later use.
template <int NW>
__device__ __forceinline__ void token_rank_mask(const int64_t *__restrict__ row, int K, int E,
                                                int epr, int epr_shift, uint64_t (&m)[NW],
                                                int64_t (&ids0)[kIdChunk])
{
#pragma unroll
    for (int w = 0; w < NW; ++w)
        m[w] = 0;
    load_ids(row, 0, K, ids0);
    add_ranks<NW>(ids0, E, epr, epr_shift, m);
    for (int k0 = kIdChunk; k0 < K; k0 += kIdChunk) {
        int64_t ids[kIdChunk];
        load_ids(row, k0, K, ids);
        add_ranks<NW>(ids, E, epr, epr_shift, m);
    }
}

// Transpose of a 64 x 64 bit matrix held one row per lane (bit j of lane i
// = entry (i, j)): afterwards lane j holds column j.  Six butterfly stages,
// each exchanging the off-diagonal halves of 2s x 2s blocks with lane ^ s.
__device__ __forceinline__ uint64_t wave_transpose64(uint64_t x)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t keep[6] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull, 0x00FF00FF00FF00FFull,
                              0x0F0F0F0F0F0F0F0Full, 0x3333333333333333ull, 0x5555555555555555ull};
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int sft = 32 >> i;
        const uint64_t lo = keep[i];  // columns c with (c & sft) == 0
        const uint64_t y = __shfl_xor((unsigned long long)x, sft, kWave);
        x = (lane & sft) ? ((x & ~lo) | ((y & ~lo) >> sft)) : ((x & lo) | ((y & lo) << sft));
    }
    return x;
}

template <int NW>
__device__ __forceinline__ void keep_live(const uint64_t *s_live, uint64_t (&m)[NW])
{
#pragma unroll
    for (int w = 0; w < NW; ++w)
        m[w] &= s_live[w];
}

__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(v, o, kWave);
        if (lane >= o)
            v += n;
    }
    return v;
}

// Count.  Every block (512 tokens = 8 waves): one ballot per rank gives each
// wave's membership mask of that rank; the block turns the 8 waves'
// popcounts into within-block offsets (LDS) and publishes masks, offsets,
// its per-rank totals and its LDS expert histogram.
// The count of block `blk` (BC tokens, BC threads); the body of
// layout_count_kernel and of the count units of layout_fused_kernel.
template <int NW, int BC>
__device__ __forceinline__ void count_body(
    int blk, const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask, int T,
    int K, int E, int R, int epr, int epr_shift, int nW, uint64_t *__restrict__ wave_mask,
    int32_t *__restrict__ wave_base, int32_t *__restrict__ blk_count,
    int32_t *__restrict__ blk_ecount)
{
    constexpr int kWaves = BC / kWave;
    extern __shared__ int32_t s_ecount[];  // [E]
    __shared__ int32_t s_wcnt[kWaves][kMaxRanks];
    __shared__ uint64_t s_live[NW];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int wg = blk * kWaves + wid;
    const int64_t t = int64_t(blk) * BC + tid;

    uint64_t m[NW];
    int64_t ids0[kIdChunk];
#pragma unroll
    for (int w = 0; w < NW; ++w)
        m[w] = 0;
#pragma unroll
    for (int q = 0; q < kIdChunk; ++q)
        ids0[q] = -1;
    const int64_t *row = topk_idx + t * K;
    if (t < T)
        token_rank_mask<NW>(row, K, E, epr, epr_shift, m, ids0);
    for (int i = tid; i < E; i += BC)
        s_ecount[i] = 0;
    build_live<NW>(rank_mask, R, s_live);
    __syncthreads();

    if (t < T) {
        keep_live<NW>(s_live, m);
        const bool masking = rank_mask != nullptr;
        for (int k0 = 0; k0 < K; k0 += kIdChunk) {
            int64_t ids[kIdChunk];
            if (k0 == 0) {
#pragma unroll
                for (int q = 0; q < kIdChunk; ++q)
                    ids[q] = ids0[q];
            } else {
                load_ids(row, k0, K, ids);
            }
#pragma unroll
            for (int q = 0; q < kIdChunk; ++q) {
                const int64_t e = ids[q];
                if (e >= 0 && e < E) {
                    // The token hits rank(e), so its bit in m says whether
                    // that rank is live.
                    bool live = true;
                    if (masking) {
                        const int r = rank_of(int(e), epr, epr_shift);
                        uint64_t word = 0;
#pragma unroll
                        for (int w = 0; w < NW; ++w)
                            word = (r >> 6) == w ? m[w] : word;
                        live = (word >> (r & 63)) & 1ull;
                    }
                    if (live)
                        atomicAdd(&s_ecount[int(e)], 1);
                }
            }
        }
    }

    // Lane b of the wave gets the wave's membership mask of rank 64w + b:
    // the transpose of the tokens' rank bitmasks.
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint64_t mine = wave_transpose64(m[w]);
        const int r = w * kWave + lane;
        if (r < R) {
            if (wg < nW)
                wave_mask[size_t(wg) * R + r] = mine;
            s_wcnt[wid][r] = __popcll(mine);
        }
    }
    __syncthreads();

    for (int r = tid; r < R; r += BC) {
        int acc = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_wcnt[w][r];
            const int g = blk * kWaves + w;
            if (g < nW)
                wave_base[size_t(g) * R + r] = acc;
            acc += c;
        }
        blk_count[size_t(blk) * R + r] = acc;
    }
    for (int i = tid; i < E; i += BC)
        blk_ecount[size_t(blk) * E + i] = s_ecount[i];
}

// With num_recv_host (a caller waiting for N), each block then bumps a
// done counter (ctr[2], which only grows: counted_base is its value before
// this launch), and the block that finishes last sums every block's per-rank
// counts -- N is their sum -- and stores N into that pinned host memory
// while the position kernel is still to run.
template <int NW>
__global__ __launch_bounds__(kCountBlock) void layout_count_kernel(
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask, int T, int K,
    int E, int R, int epr, int epr_shift, int nW, uint64_t *__restrict__ wave_mask,
    int32_t *__restrict__ wave_base, int32_t *__restrict__ blk_count,
    int32_t *__restrict__ blk_ecount, uint64_t *__restrict__ ctr, uint64_t counted_base,
    int64_t *num_recv_host)
{
    count_body<NW, kCountBlock>(blockIdx.x, topk_idx, rank_mask, T, K, E, R, epr, epr_shift, nW,
                                wave_mask, wave_base, blk_count, blk_ecount);
    if (num_recv_host == nullptr)
        return;
    constexpr int kWaves = kCountBlock / kWave;
    __shared__ int s_last;
    __shared__ int64_t s_part[kWaves];
    const int tid = threadIdx.x;
    __syncthreads();  // every wave's blk_count stores are done
    if (tid == 0) {
        const uint64_t before = __hip_atomic_fetch_add(&ctr[2], uint64_t(1), __ATOMIC_RELEASE,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        s_last = before - counted_base == uint64_t(gridDim.x - 1);
        if (s_last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!s_last)
        return;
    const int n = int(gridDim.x) * R;
    int64_t sum = 0;
    for (int i = tid; i < n; i += kCountBlock)
        sum += blk_count[i];
#pragma unroll
    for (int sft = kWave / 2; sft > 0; sft >>= 1)
        sum += __shfl_xor((long long)sum, sft, kWave);
    if ((tid & (kWave - 1)) == 0)
        s_part[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        int64_t N = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            N += s_part[w];
        __hip_atomic_store(num_recv_host, N, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

constexpr int kPosBlock = 256;
constexpr int kPosGrid = 512;   // split tiles while the grid stays within this
constexpr int kSelfScanBlocks = 32;  // up to this many count blocks, pos blocks scan for themselves
constexpr int kBatch = 8;

// Block-wide exclusive scan of v over ranks (R <= 2 * kPosBlock): each thread
// holds two consecutive ranks.  Writes S[r] into s_seg and returns N.
__device__ __forceinline__ int rank_exclusive_scan(const int32_t *s_tot, int32_t *s_seg, int R,
                                                   int32_t *s_wsum)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int r0 = 2 * tid;
    const int a = r0 < R ? s_tot[r0] : 0;
    const int b = r0 + 1 < R ? s_tot[r0 + 1] : 0;
    const int incl = wave_inclusive_scan(a + b);
    if (lane == kWave - 1)
        s_wsum[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPosBlock / kWave; ++w) {
        before += w < wid ? s_wsum[w] : 0;
        total += s_wsum[w];
    }
    const int ex = before + incl - (a + b);
    if (r0 < R)
        s_seg[r0] = ex;
    if (r0 + 1 < R)
        s_seg[r0 + 1] = ex + a;
    return total;
}

// Totals only the layout as a whole knows: per-rank and per-expert counts,
// rank_prefix_matrix, N, and the channel entries at the last token.
__device__ void write_totals(int T, int E, int R, int C, int nB, const int32_t *s_tot,
                             const int32_t *s_seg, const int32_t *__restrict__ blk_ecount,
                             int32_t *__restrict__ num_tokens_per_rank,
                             int32_t *__restrict__ num_tokens_per_expert,
                             int32_t *__restrict__ rank_prefix_matrix,
                             int32_t *__restrict__ channel_prefix_matrix,
                             int32_t *__restrict__ recv_channel_prefix_matrix,
                             int64_t *__restrict__ num_recv, int64_t *num_recv_host, int N,
                             int nthreads)
{
    const int tid = threadIdx.x;
    for (int r = tid; r < R; r += nthreads) {
        num_tokens_per_rank[r] = s_tot[r];
        rank_prefix_matrix[r] = s_seg[r] + s_tot[r];
        recv_channel_prefix_matrix[size_t(r) * C] = 0;
    }
    if (tid == 0) {
        *num_recv = N;
        // the host copy (pinned, coherent) that a caller waiting for N polls
        if (num_recv_host != nullptr)
            __hip_atomic_store(num_recv_host, int64_t(N), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
    }
    for (int e = tid; e < E; e += nthreads) {
        int sum = 0;
        for (int b0 = 0; b0 < nB; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                c[i] = b0 + i < nB ? blk_ecount[size_t(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                sum += c[i];
        }
        num_tokens_per_expert[e] = sum;
    }
    const int per = T > 0 ? (T + C - 1) / C : 1;
    const int c0 = T > 0 ? (T + per - 1) / per - 1 : 0;  // first c with end(c) == T
    const int ntail = C - c0;
    for (int i = tid; i < R * ntail; i += nthreads) {
        const int r = i / ntail;
        const int c = c0 + i % ntail;
        channel_prefix_matrix[size_t(r) * C + c] = s_tot[r];
        if (c + 1 < C)
            recv_channel_prefix_matrix[size_t(r) * C + c + 1] = s_tot[r];
    }
}

// Scan for large token counts (more than kSelfScanBlocks count blocks): one
// block turns the block totals into exclusive bases in place and writes the
// totals.  Also the whole layout of an empty token range.
__global__ __launch_bounds__(kPosBlock) void layout_scan_kernel(
    int T, int E, int R, int C, int nB, int32_t *__restrict__ blk_count,
    const int32_t *__restrict__ blk_ecount, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix_matrix,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix,
    int64_t *__restrict__ num_recv, int64_t *num_recv_host)
{
    __shared__ int32_t s_tot[kMaxRanks];
    __shared__ int32_t s_seg[kMaxRanks];
    __shared__ int32_t s_wsum[kPosBlock / kWave];
    for (int r = threadIdx.x; r < R; r += kPosBlock) {
        int carry = 0;
        for (int b0 = 0; b0 < nB; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                c[i] = b0 + i < nB ? blk_count[size_t(b0 + i) * R + r] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (b0 + i < nB)
                    blk_count[size_t(b0 + i) * R + r] = carry;
                carry += c[i];
            }
        }
        s_tot[r] = T > 0 ? carry : 0;
    }
    __syncthreads();
    const int N = rank_exclusive_scan(s_tot, s_seg, R, s_wsum);
    __syncthreads();
    write_totals(T, E, R, C, T > 0 ? nB : 0, s_tot, s_seg, blk_ecount, num_tokens_per_rank,
                 num_tokens_per_expert, rank_prefix_matrix, channel_prefix_matrix,
                 recv_channel_prefix_matrix, num_recv, num_recv_host, N, kPosBlock);
}

// Positions of one 64-token tile, or of a 2^sub_shift-th part of it (small
// grids split their tiles so that more of the chip works).  With kSelfScan
// the workgroup first sums the count blocks' per-rank totals itself (all
// loads of a batch issued before any add): those before its own block give
// its bases, all of them give the segment starts S[r]; the first workgroup
// also writes the totals.  Otherwise the bases were made by
// layout_scan_kernel.
//
// The (token, rank) cells of the workgroup's tokens are then spread flat over
// its lanes: each cell's position is its tile base plus a popcount of the
// rank's membership mask below the token, so there is no loop-carried
// dependence, and consecutive lanes write consecutive entries of every [T][R]
// row (send_head, is_token_in_rank).  Finally groups of lanes emit each
// token's destination rows in ascending rank order, the list the pack and
// reduce kernels read.
template <int NW, bool kSelfScan, int BC>
__device__ __forceinline__ void pos_body(
    int vb, int T, int E, int R, int C, int kmax, int nB, int sub_shift,
    const uint64_t *__restrict__ wave_mask, const int32_t *__restrict__ wave_base,
    const int32_t *__restrict__ blk_count, const int32_t *__restrict__ blk_ecount,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ send_head,
    int32_t *__restrict__ recv_src_idx, int32_t *__restrict__ dst_row,
    int32_t *__restrict__ dst_rank, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix_matrix,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix,
    int64_t *__restrict__ num_recv, int64_t *num_recv_host)
{
    __shared__ uint64_t s_mask[NW * kWave];
    __shared__ int32_t s_seg[NW * kWave];  // S[r]
    __shared__ int32_t s_off[NW * kWave];  // position of this tile's first hit inside segment r
    __shared__ int32_t s_tot[NW * kWave];
    __shared__ int32_t s_wsum[kPosBlock / kWave];
    __shared__ uint64_t s_tokm[NW][kWave];  // live-rank bitmask of each token of the tile
    const int tid = threadIdx.x;
    // 2^sub_shift workgroups (1, 2 or 4) share a tile, sub_tok tokens each
    // (powers of two throughout: shifts and masks, no integer division)
    const int wg = vb >> sub_shift;  // the 64-token tile
    const int sub = vb & ((1 << sub_shift) - 1);
    const int sub_tok = kWave >> sub_shift;
    const int blk = wg / (BC / kWave);  // its count block
    const int64_t t0 = int64_t(wg) * kWave;
    const int ntok = int(T - t0 < kWave ? T - t0 : kWave);
    // this workgroup's tokens of the tile: [lo, hi)
    const int lo = sub * sub_tok;
    const int hi = lo + sub_tok < ntok ? lo + sub_tok : ntok;
    if (lo >= hi)
        return;  // uniform over the workgroup, before any barrier

    // Per-rank state of the tile.  The count kernel stored, for each rank, the
    // mask of the tile's tokens that hit it (ranks masked at the time already
    // cleared).  The loop runs over whole 64-rank words, so each wave also
    // transposes the words it loaded: that gives every token its mask of
    // ranks, without reading the top-k ids again.
    for (int r = tid; r < NW * kWave; r += kPosBlock) {
        uint64_t bm = 0;
        if (r < R) {
            bm = wave_mask[size_t(wg) * R + r];
            s_mask[r] = bm;
            int before = 0, tot = 0;
            if (kSelfScan) {
                for (int b0 = 0; b0 < nB; b0 += kBatch) {
                    int c[kBatch];
#pragma unroll
                    for (int i = 0; i < kBatch; ++i)
                        c[i] = b0 + i < nB ? blk_count[size_t(b0 + i) * R + r] : 0;
#pragma unroll
                    for (int i = 0; i < kBatch; ++i) {
                        before += b0 + i < blk ? c[i] : 0;
                        tot += c[i];
                    }
                }
                s_tot[r] = tot;
            } else {
                before = blk_count[size_t(blk) * R + r];
            }
            s_off[r] = before + wave_base[size_t(wg) * R + r];
        }
        s_tokm[r >> 6][r & (kWave - 1)] = wave_transpose64(bm);
    }
    __syncthreads();
    if (kSelfScan) {
        const int N = rank_exclusive_scan(s_tot, s_seg, R, s_wsum);
        __syncthreads();
        if (wg == 0 && sub == 0)
            write_totals(T, E, R, C, nB, s_tot, s_seg, blk_ecount, num_tokens_per_rank,
                         num_tokens_per_expert, rank_prefix_matrix, channel_prefix_matrix,
                         recv_channel_prefix_matrix, num_recv, num_recv_host, N, kPosBlock);
    } else {
        for (int r = tid; r < R; r += kPosBlock)
            s_seg[r] = r > 0 ? rank_prefix_matrix[r - 1] : 0;
        __syncthreads();
    }

    // Flat walk over the tile's cells, (token, rank) row-major, so that
    // consecutive lanes write consecutive entries of the [T][R] rows.  With R
    // a multiple of 4 a lane takes 4 ranks: one 16-byte send_head store and
    // one 4-byte is_token_in_rank store.
    if ((R & 3) == 0) {
        const int G = R >> 2;
        const int items = (hi - lo) * G;
        const int dt = kPosBlock / G, dg = kPosBlock % G;
        int tl = lo + tid / G, g = tid % G;
        for (int i = tid; i < items; i += kPosBlock) {
            const int64_t t = t0 + tl;
            const uint64_t below = (1ull << tl) - 1ull;
            int4 sh;
            uint32_t in4 = 0;
            int *shp = reinterpret_cast<int *>(&sh);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 4 * g + q;
                const uint64_t b = s_mask[r];
                const bool hit = (b >> tl) & 1ull;
                shp[q] = hit ? s_off[r] + __popcll(b & below) : -1;
                in4 |= (hit ? 1u : 0u) << (8 * q);
            }
            *reinterpret_cast<int4 *>(send_head + size_t(t) * R + 4 * g) = sh;
            *reinterpret_cast<uint32_t *>(is_token_in_rank + size_t(t) * R + 4 * g) = in4;
            tl += dt;
            g += dg;
            if (g >= G) {
                g -= G;
                ++tl;
            }
        }
    } else {
        const int cells = (hi - lo) * R;
        const int dt = kPosBlock / R, dr = kPosBlock % R;
        int tl = lo + tid / R, r = tid % R;
        for (int i = tid; i < cells; i += kPosBlock) {
            const uint64_t b = s_mask[r];
            const bool hit = (b >> tl) & 1ull;
            const int pos = s_off[r] + __popcll(b & ((1ull << tl) - 1ull));
            const int64_t t = t0 + tl;
            send_head[size_t(t) * R + r] = hit ? pos : -1;
            is_token_in_rank[size_t(t) * R + r] = hit ? 1 : 0;
            tl += dt;
            r += dr;
            if (r >= R) {
                r -= R;
                ++tl;
            }
        }
    }

    // Channel ends at this workgroup's tokens: hits of rank r before the
    // boundary token.
    const int per = (T + C - 1) / C;
    int64_t boundary = ((t0 + lo + per - 1) / per) * per;  // smallest multiple of per >= t0 + lo
    if (boundary == 0)
        boundary = per;
    for (; boundary < t0 + hi; boundary += per) {
        const int bl = int(boundary - t0);
        const int64_t c = boundary / per - 1;
        for (int rr = tid; rr < R; rr += kPosBlock) {
            const int cnt = s_off[rr] + __popcll(s_mask[rr] & ((1ull << bl) - 1ull));
            channel_prefix_matrix[size_t(rr) * C + c] = cnt;
            recv_channel_prefix_matrix[size_t(rr) * C + c + 1] = cnt;
        }
    }

    // Each token's destination rows in ascending rank order (and the inverse
    // map recv_src_idx): sub_tok lanes per token group, and group p of the
    // workgroup writes the entries j with j % parts == p.
    {
        const int parts = (kPosBlock / kWave) << sub_shift;  // kPosBlock / sub_tok
        const int tl = lo + (tid & (sub_tok - 1));
        const int part = tid >> (6 - sub_shift);
        if (tl < hi) {
            const int64_t t = t0 + tl;
            const uint64_t below = (1ull << tl) - 1ull;
            int j = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                uint64_t mm = s_tokm[w][tl];
                while (mm) {
                    const int bit = __ffsll((unsigned long long)mm) - 1;
                    mm &= mm - 1;
                    if ((j & (parts - 1)) == part) {
                        const int rr = w * kWave + bit;
                        const int row = s_seg[rr] + s_off[rr] + __popcll(s_mask[rr] & below);
                        dst_row[size_t(t) * kmax + j] = row;
                        dst_rank[size_t(t) * kmax + j] = rr;
                        recv_src_idx[row] = int32_t(t);
                    }
                    ++j;
                }
            }
            for (; j < kmax; ++j) {
                if ((j & (parts - 1)) == part) {
                    dst_row[size_t(t) * kmax + j] = -1;
                    dst_rank[size_t(t) * kmax + j] = -1;
                }
            }
        }
    }
}

template <int NW, bool kSelfScan>
__global__ __launch_bounds__(kPosBlock) void layout_pos_kernel(
    int T, int E, int R, int C, int kmax, int nB, int sub_shift,
    const uint64_t *__restrict__ wave_mask, const int32_t *__restrict__ wave_base,
    const int32_t *__restrict__ blk_count, const int32_t *__restrict__ blk_ecount,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ send_head,
    int32_t *__restrict__ recv_src_idx, int32_t *__restrict__ dst_row,
    int32_t *__restrict__ dst_rank, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix_matrix,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix,
    int64_t *__restrict__ num_recv, int64_t *num_recv_host)
{
    pos_body<NW, kSelfScan, kCountBlock>(
        blockIdx.x, T, E, R, C, kmax, nB, sub_shift, wave_mask, wave_base, blk_count, blk_ecount,
        is_token_in_rank, send_head, recv_src_idx, dst_row, dst_rank, num_tokens_per_rank,
        num_tokens_per_expert, rank_prefix_matrix, channel_prefix_matrix,
        recv_channel_prefix_matrix, num_recv, num_recv_host);
}

// One-launch layout for up to kSelfScanBlocks count blocks of kFusedCount
// tokens.  Every workgroup first takes a ticket from a counter in the
// handle's arena: the first nB tickets of this launch are count units, the
// rest position units, so work is handed out in the order workgroups start,
// whatever order the hardware starts them in.  A count unit publishes its
// block (one device-scope release) and bumps the done counter; a position
// unit polls that counter with relaxed loads (an acquire at every poll would
// invalidate this XCD's L2 under the count units still running) until all
// nB count units of this launch are done, then takes one device-scope
// acquire and runs as layout_pos_kernel would.  Count units never wait, and
// a ticket is only taken by a workgroup that is running, so the wait always
// ends however few workgroups fit on the chip at once.  (A bound on the
// wait, seconds, far beyond any real layout, sets a sticky flag and skips
// the unit's writes rather than hang.)
// The counters only grow: the host keeps, per arena, how many tickets and
// done marks earlier launches used and passes those bases in, so nothing
// has to reset them (and no workgroup has to fence on its way out).
constexpr int kFusedCount = 256;  // tokens (and threads) of a fused count unit
constexpr unsigned kFusedMaxPolls = 1u << 22;

template <int NW>
__global__ __launch_bounds__(kPosBlock) void layout_fused_kernel(
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask, int T, int K,
    int E, int R, int C, int epr, int epr_shift, int kmax, int nW, int nB, int sub_shift,
    uint64_t *__restrict__ ctr, uint64_t ticket_base, uint64_t done_base,
    uint64_t *__restrict__ wave_mask, int32_t *__restrict__ wave_base,
    int32_t *__restrict__ blk_count, int32_t *__restrict__ blk_ecount,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ send_head,
    int32_t *__restrict__ recv_src_idx, int32_t *__restrict__ dst_row,
    int32_t *__restrict__ dst_rank, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix_matrix,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix,
    int64_t *__restrict__ num_recv, int64_t *num_recv_host)
{
    static_assert(kFusedCount == kPosBlock, "one workgroup shape for both unit kinds");
    __shared__ int s_ticket;
    __shared__ int s_ready;
    const int tid = threadIdx.x;
    if (tid == 0)
        s_ticket = int(__hip_atomic_fetch_add(&ctr[0], uint64_t(1), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) -
                       ticket_base);
    __syncthreads();
    const int ticket = s_ticket;
    if (ticket < nB) {
        count_body<NW, kFusedCount>(ticket, topk_idx, rank_mask, T, K, E, R, epr, epr_shift, nW,
                                    wave_mask, wave_base, blk_count, blk_ecount);
        __syncthreads();  // every wave's stores have reached L2
        if (tid == 0)
            __hip_atomic_fetch_add(&ctr[1], uint64_t(1), __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
    } else if (ticket < int(gridDim.x)) {
        if (tid == 0) {
            unsigned polls = 0;
            int ready = 1;
            while (__hip_atomic_load(&ctr[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                       done_base <
                   uint64_t(nB)) {
                __builtin_amdgcn_s_sleep(2);
                if (++polls == kFusedMaxPolls) {
                    __hip_atomic_store(&ctr[3], uint64_t(1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    ready = 0;
                    break;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_ready = ready;
        }
        __syncthreads();
        // without all counts the positions could point anywhere: write none
        if (s_ready)
            pos_body<NW, true, kFusedCount>(
                ticket - nB, T, E, R, C, kmax, nB, sub_shift, wave_mask, wave_base, blk_count,
                blk_ecount, is_token_in_rank, send_head, recv_src_idx, dst_row, dst_rank,
                num_tokens_per_rank, num_tokens_per_expert, rank_prefix_matrix,
                channel_prefix_matrix, recv_channel_prefix_matrix, num_recv, num_recv_host);
    }
}

// log2 of the workgroups per tile of the position kernel: a small grid
// leaves most of the chip idle, so its tiles are split (each part repeats
// the tile's cheap per-rank setup); a grid that already fills the chip is not.
int pos_split_shift(int nW)
{
    int sh = 2;  // at most 4 workgroups per tile
    while (sh > 0 && (int64_t(nW) << sh) > kPosGrid)
        --sh;
    return sh;
}

template <int NW>
hipError_t launch_layout_nw(const LayoutShape &s, const int64_t *topk_idx,
                            const int32_t *rank_mask, const LayoutBufs &b,
                            int64_t *num_recv_host, LayoutCounters &lc, hipStream_t stream)
{
    const int epr_shift = (s.epr & (s.epr - 1)) == 0 ? __builtin_ctz(unsigned(s.epr)) : -1;
    const int sub_shift = pos_split_shift(s.nW);
    if (s.fused) {
        const unsigned grid = unsigned(s.nB) + (unsigned(s.nW) << sub_shift);
        hipLaunchKernelGGL(layout_fused_kernel<NW>, dim3(grid), dim3(kPosBlock),
                           size_t(s.E) * sizeof(int32_t), stream, topk_idx, rank_mask, s.T, s.K,
                           s.E, s.R, s.C, s.epr, epr_shift, s.kmax, s.nW, s.nB, sub_shift,
                           b.layout_ctr, lc.tickets, lc.done, b.wave_mask, b.wave_base,
                           b.blk_count, b.blk_ecount, b.is_token_in_rank, b.send_head,
                           b.recv_src_idx, b.dst_row, b.dst_rank, b.num_tokens_per_rank,
                           b.num_tokens_per_expert, b.rank_prefix_matrix, b.channel_prefix_matrix,
                           b.recv_channel_prefix_matrix, b.num_recv, num_recv_host);
        const hipError_t e = hipGetLastError();
        if (e == hipSuccess) {
            lc.tickets += grid;
            lc.done += unsigned(s.nB);
        }
        return e;
    }
    // N for the host: from the count kernel when there is one, else (no
    // tokens) from the scan kernel, which then writes the whole layout
    if (s.T > 0) {
        hipLaunchKernelGGL(layout_count_kernel<NW>, dim3(s.nB), dim3(kCountBlock),
                           size_t(s.E) * sizeof(int32_t), stream, topk_idx, rank_mask, s.T, s.K, s.E, s.R,
                           s.epr, epr_shift, s.nW, b.wave_mask, b.wave_base, b.blk_count,
                           b.blk_ecount, b.layout_ctr, lc.counted, num_recv_host);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (num_recv_host != nullptr)
            lc.counted += unsigned(s.nB);
    }
    int64_t *const totals_host = s.T > 0 ? nullptr : num_recv_host;
    const bool self_scan = s.T > 0 && s.nB <= kSelfScanBlocks;
    if (!self_scan)
        hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kPosBlock), 0, stream, s.T, s.E, s.R,
                           s.C, s.nB, b.blk_count, b.blk_ecount, b.num_tokens_per_rank,
                           b.num_tokens_per_expert, b.rank_prefix_matrix, b.channel_prefix_matrix,
                           b.recv_channel_prefix_matrix, b.num_recv, totals_host);
    auto pos_kernel = self_scan ? layout_pos_kernel<NW, true> : layout_pos_kernel<NW, false>;
    if (s.T > 0)
        hipLaunchKernelGGL(pos_kernel, dim3(unsigned(s.nW) << sub_shift), dim3(kPosBlock), 0, stream,
                           s.T, s.E, s.R, s.C, s.kmax, s.nB, sub_shift, b.wave_mask, b.wave_base, b.blk_count,
                           b.blk_ecount, b.is_token_in_rank, b.send_head, b.recv_src_idx,
                           b.dst_row, b.dst_rank, b.num_tokens_per_rank, b.num_tokens_per_expert,
                           b.rank_prefix_matrix, b.channel_prefix_matrix,
                           b.recv_channel_prefix_matrix, b.num_recv, totals_host);
    return hipGetLastError();
}

std::atomic<int> g_layout_mode{0};  // 0 automatic (= 1), 1 two kernels, 2 one launch when it fits

}  // namespace

bool set_layout_tuning(int mode)
{
    if (mode < 0 || mode > 2)
        return false;
    g_layout_mode = mode;
    return true;
}

LayoutShape layout_shape(const ep_dims &d, bool allow_fused)
{
    LayoutShape s;
    s.T = d.num_tokens;
    s.K = d.num_topk;
    s.E = d.num_experts;
    s.R = d.num_ranks;
    s.C = d.num_channels;
    s.epr = s.E / s.R;
    s.kmax = s.K < s.R ? s.K : s.R;
    s.nW = (s.T + kWave - 1) / kWave;
    // One launch only when asked for (and while its position units can sum
    // all count blocks themselves): its grid-wide wait costs more than the
    // second launch it saves (13.4 against 4.2 + 5.9 us at 4096 tokens).
    const int64_t fused_blocks = (int64_t(s.T) + kFusedCount - 1) / kFusedCount;
    s.fused = allow_fused && g_layout_mode.load() == 2 && s.T > 0 &&
              fused_blocks <= kSelfScanBlocks;
    const int cb = s.fused ? kFusedCount : kCountBlock;
    s.nB = s.T > 0 ? (s.T + cb - 1) / cb : 1;
    return s;
}

size_t layout_arena_bytes(const LayoutShape &s, size_t off[kArenaFields])
{
    const size_t T = size_t(s.T), R = size_t(s.R), E = size_t(s.E), C = size_t(s.C);
    const size_t km = size_t(s.kmax), nW = size_t(s.nW), nB = size_t(s.nB);
    // field 0, the one-launch layout's counters, is first so that it sits at
    // the same place for every shape that reuses the arena
    const size_t sizes[kArenaFields] = {
        kLayoutCtrBytes, R * 4,      E * 4,      T * R,      R * 4,      R * C * 4,
        R * C * 4,       T * R * 4,  T * km * 4, T * km * 4, T * km * 4, nW * R * 8,
        nW * R * 4,      nB * R * 4, nB * E * 4, 8,          16,
    };
    size_t cur = 0;
    for (int i = 0; i < kArenaFields; ++i) {
        off[i] = cur;
        cur += (sizes[i] + 255) & ~size_t(255);
    }
    return cur;
}

LayoutBufs layout_bufs_at(void *base, const size_t off[kArenaFields])
{
    char *p = static_cast<char *>(base);
    LayoutBufs b;
    b.layout_ctr = reinterpret_cast<uint64_t *>(p + off[0]);
    b.num_tokens_per_rank = reinterpret_cast<int32_t *>(p + off[1]);
    b.num_tokens_per_expert = reinterpret_cast<int32_t *>(p + off[2]);
    b.is_token_in_rank = reinterpret_cast<uint8_t *>(p + off[3]);
    b.rank_prefix_matrix = reinterpret_cast<int32_t *>(p + off[4]);
    b.channel_prefix_matrix = reinterpret_cast<int32_t *>(p + off[5]);
    b.recv_channel_prefix_matrix = reinterpret_cast<int32_t *>(p + off[6]);
    b.send_head = reinterpret_cast<int32_t *>(p + off[7]);
    b.recv_src_idx = reinterpret_cast<int32_t *>(p + off[8]);
    b.dst_row = reinterpret_cast<int32_t *>(p + off[9]);
    b.dst_rank = reinterpret_cast<int32_t *>(p + off[10]);
    b.wave_mask = reinterpret_cast<uint64_t *>(p + off[11]);
    b.wave_base = reinterpret_cast<int32_t *>(p + off[12]);
    b.blk_count = reinterpret_cast<int32_t *>(p + off[13]);
    b.blk_ecount = reinterpret_cast<int32_t *>(p + off[14]);
    b.num_recv = reinterpret_cast<int64_t *>(p + off[15]);
    b.topk_hash = reinterpret_cast<uint64_t *>(p + off[16]);
    return b;
}

hipError_t launch_layout(const LayoutShape &s, const int64_t *topk_idx, const int32_t *rank_mask,
                         const LayoutBufs &b, int64_t *num_recv_host, LayoutCounters &lc,
                         hipStream_t stream)
{
    if (log_enabled())
        log_launch("layout T=%d K=%d E=%d R=%d C=%d: count blocks=%d pos blocks=%d%s%s%s", s.T,
                   s.K, s.E, s.R, s.C, s.nB, s.nW, s.fused ? " one-launch" : "",
                   !s.fused && s.nB > kSelfScanBlocks ? " +scan" : "",
                   rank_mask != nullptr ? " +mask" : "");
    switch ((s.R + kWave - 1) / kWave) {
    case 1: return launch_layout_nw<1>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    case 2: return launch_layout_nw<2>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    case 3: return launch_layout_nw<3>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    case 4: return launch_layout_nw<4>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    case 5:
    case 6: return launch_layout_nw<6>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    case 7:
    case 8: return launch_layout_nw<8>(s, topk_idx, rank_mask, b, num_recv_host, lc, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ep

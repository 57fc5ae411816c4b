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
// Three launches, all stream-ordered:
//   count: one wavefront per 64 tokens.  Each lane builds its token's rank
//          bitmask; one ballot per rank gives the wave's 64-bit membership
//          mask for that rank, whose popcount is the wave's count.  Expert
//          counts go to an LDS-privatised histogram per block.
//   scan:  one block.  Per rank, an exclusive scan of the wave counts (one
//          wavefront per rank); a block scan of the rank totals gives
//          rank_prefix_matrix; expert totals; the channel entries that end at
//          the last token.
//   pos:   one wavefront per 64 tokens again.  Lanes take ranks and walk the
//          wave's tokens, so every [T][R] row (send_head, is_token_in_rank)
//          is written by contiguous lanes; then lanes take tokens and emit
//          each token's destination rows in ascending rank order, the list
//          the pack and reduce kernels read.
// Positions come from ballots and scans, never from atomics, so every output
// is deterministic and segments are in token order.

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLayoutBlock = 256;  // 4 wavefronts = 256 tokens per block

template <int NW>
__device__ __forceinline__ void token_rank_mask(const int64_t *__restrict__ row, int K, int E,
                                                int epr, uint64_t (&m)[NW])
{
#pragma unroll
    for (int w = 0; w < NW; ++w)
        m[w] = 0;
    for (int k = 0; k < K; ++k) {
        const int64_t e = row[k];
        if (e >= 0 && e < E) {
            const int r = int(e) / epr;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if ((r >> 6) == w)
                    m[w] |= 1ull << (r & 63);
        }
    }
}

template <int NW>
__global__ __launch_bounds__(kLayoutBlock) void layout_count_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int epr, int nW,
    uint64_t *__restrict__ wave_mask, int32_t *__restrict__ wave_count,
    int32_t *__restrict__ blk_ecount)
{
    extern __shared__ int32_t s_ecount[];  // [E]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wg = blockIdx.x * (kLayoutBlock / kWave) + (tid >> 6);
    const int64_t t = int64_t(blockIdx.x) * kLayoutBlock + tid;

    for (int i = tid; i < E; i += kLayoutBlock)
        s_ecount[i] = 0;
    __syncthreads();

    uint64_t m[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w)
        m[w] = 0;
    if (t < T) {
        const int64_t *row = topk_idx + t * K;
        token_rank_mask<NW>(row, K, E, epr, m);
        for (int k = 0; k < K; ++k) {
            const int64_t e = row[k];
            if (e >= 0 && e < E)
                atomicAdd(&s_ecount[int(e)], 1);
        }
    }

    if (wg < nW) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            uint64_t mine = 0;
            for (int b = 0; b < kWave; ++b) {
                const int r = w * kWave + b;
                if (r >= R)
                    break;
                const uint64_t bal = wave_ballot((m[w] >> b) & 1ull);
                if (lane == b)
                    mine = bal;
            }
            const int r = w * kWave + lane;
            if (r < R) {
                wave_mask[size_t(wg) * R + r] = mine;
                wave_count[size_t(r) * nW + wg] = __popcll(mine);
            }
        }
    }

    __syncthreads();
    for (int i = tid; i < E; i += kLayoutBlock)
        blk_ecount[size_t(blockIdx.x) * E + i] = s_ecount[i];
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

constexpr int kScanBlock = 1024;

__global__ __launch_bounds__(kScanBlock) void layout_scan_kernel(
    int T, int E, int R, int C, int nW, int nB, int32_t *__restrict__ wave_count,
    const int32_t *__restrict__ blk_ecount, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix_matrix,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix,
    int64_t *__restrict__ num_recv)
{
    __shared__ int32_t s_tot[kMaxRanks];
    __shared__ int32_t s_wsum[kScanBlock / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    constexpr int kWaves = kScanBlock / kWave;

    // Per rank: exclusive scan of the wave counts over waves, in place.
    for (int r = wid; r < R; r += kWaves) {
        int32_t *row = wave_count + size_t(r) * nW;
        int carry = 0;
        for (int base = 0; base < nW; base += kWave) {
            const int i = base + lane;
            const int v = i < nW ? row[i] : 0;
            const int incl = wave_inclusive_scan(v);
            if (i < nW)
                row[i] = carry + incl - v;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            s_tot[r] = carry;
    }
    __syncthreads();

    // Rank totals and their inclusive prefix (R <= 512 < block size).
    const int v = tid < R ? s_tot[tid] : 0;
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1)
        s_wsum[wid] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wid; ++w)
        before += s_wsum[w];
    if (tid < R) {
        num_tokens_per_rank[tid] = v;
        rank_prefix_matrix[tid] = before + incl;
        if (tid == R - 1)
            *num_recv = before + incl;
    }

    // Expert totals over the count blocks.
    for (int e = tid; e < E; e += kScanBlock) {
        int s = 0;
        for (int b = 0; b < nB; ++b)
            s += blk_ecount[size_t(b) * E + e];
        num_tokens_per_expert[e] = s;
    }

    // Channels ending at the last token hold the rank totals; channel 0 of the
    // exclusive matrix is 0.  The other entries sit on token boundaries and
    // are written by the position kernel.
    const int per = T > 0 ? (T + C - 1) / C : 1;
    const int c0 = T > 0 ? (T + per - 1) / per - 1 : 0;  // first c with end(c) == T
    const int ntail = C - c0;
    for (int i = tid; i < R * ntail; i += kScanBlock) {
        const int r = i / ntail;
        const int c = c0 + i % ntail;
        const int tot = s_tot[r];
        channel_prefix_matrix[size_t(r) * C + c] = tot;
        if (c + 1 < C)
            recv_channel_prefix_matrix[size_t(r) * C + c + 1] = tot;
    }
    for (int r = tid; r < R; r += kScanBlock)
        recv_channel_prefix_matrix[size_t(r) * C] = 0;
}

template <int NW>
__global__ __launch_bounds__(kLayoutBlock) void layout_pos_kernel(
    const int64_t *__restrict__ topk_idx, int T, int K, int E, int R, int C, int epr, int kmax,
    int nW, const uint64_t *__restrict__ wave_mask, const int32_t *__restrict__ wave_base,
    const int32_t *__restrict__ rank_prefix_matrix, uint8_t *__restrict__ is_token_in_rank,
    int32_t *__restrict__ send_head, int32_t *__restrict__ recv_src_idx,
    int32_t *__restrict__ dst_row, int32_t *__restrict__ dst_rank,
    int32_t *__restrict__ channel_prefix_matrix, int32_t *__restrict__ recv_channel_prefix_matrix)
{
    constexpr int kWavesPerBlock = kLayoutBlock / kWave;
    __shared__ uint64_t s_mask[kWavesPerBlock][NW * kWave];
    __shared__ int32_t s_row0[kWavesPerBlock][NW * kWave];  // S[r] + wave base of r
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wib = tid >> 6;
    const int wg = blockIdx.x * kWavesPerBlock + wib;
    const bool wave_live = wg < nW;
    const int64_t t0 = int64_t(wg) * kWave;

    if (wave_live) {
        for (int r = lane; r < R; r += kWave) {
            s_mask[wib][r] = wave_mask[size_t(wg) * R + r];
            const int seg = r > 0 ? rank_prefix_matrix[r - 1] : 0;
            s_row0[wib][r] = seg + wave_base[size_t(r) * nW + wg];
        }
    }
    __syncthreads();
    if (!wave_live)
        return;

    // Lanes = ranks: walk the wave's tokens in order.
    const int ntok = int(T - t0 < kWave ? T - t0 : kWave);
    const int per = (T + C - 1) / C;
    int64_t first_boundary = ((t0 + per - 1) / per) * per;  // smallest multiple of per >= t0
    if (first_boundary == 0)
        first_boundary = per;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int r = w * kWave + lane;
        const bool act = r < R;
        const uint64_t b = act ? s_mask[wib][r] : 0;
        const int row0 = act ? s_row0[wib][r] : 0;
        const int seg = act ? (r > 0 ? rank_prefix_matrix[r - 1] : 0) : 0;
        int pos = row0 - seg;  // position inside segment r of the next hit
        int64_t boundary = first_boundary;
        for (int tl = 0; tl < ntok; ++tl) {
            const int64_t t = t0 + tl;
            const bool hit = (b >> tl) & 1ull;
            if (t == boundary) {  // end of channel t/per - 1, which is < T
                if (act) {
                    const int64_t c = t / per - 1;
                    channel_prefix_matrix[size_t(r) * C + c] = pos;
                    recv_channel_prefix_matrix[size_t(r) * C + c + 1] = pos;
                }
                boundary += per;
            }
            if (act) {
                send_head[size_t(t) * R + r] = hit ? pos : -1;
                is_token_in_rank[size_t(t) * R + r] = hit ? 1 : 0;
                if (hit)
                    recv_src_idx[seg + pos] = int32_t(t);
            }
            pos += hit ? 1 : 0;
        }
    }

    // Lanes = tokens: each token's destination rows, ascending rank.
    const int64_t t = t0 + lane;
    if (t < T) {
        uint64_t m[NW];
        token_rank_mask<NW>(topk_idx + t * K, K, E, epr, m);
        const uint64_t below = lanemask_lt();
        int j = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            uint64_t mm = m[w];
            while (mm) {
                const int bit = __ffsll((unsigned long long)mm) - 1;
                mm &= mm - 1;
                const int r = w * kWave + bit;
                const int row = s_row0[wib][r] + __popcll(s_mask[wib][r] & below);
                dst_row[size_t(t) * kmax + j] = row;
                dst_rank[size_t(t) * kmax + j] = r;
                ++j;
            }
        }
        for (; j < kmax; ++j) {
            dst_row[size_t(t) * kmax + j] = -1;
            dst_rank[size_t(t) * kmax + j] = -1;
        }
    }
}

template <int NW>
hipError_t launch_layout_nw(const LayoutShape &s, const int64_t *topk_idx, const LayoutBufs &b,
                            hipStream_t stream)
{
    if (s.T > 0) {
        hipLaunchKernelGGL(layout_count_kernel<NW>, dim3(s.nB), dim3(kLayoutBlock),
                           size_t(s.E) * sizeof(int32_t), stream, topk_idx, s.T, s.K, s.E, s.R,
                           s.epr, s.nW, b.wave_mask, b.wave_count, b.blk_ecount);
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanBlock), 0, stream, s.T, s.E, s.R,
                       s.C, s.nW, s.nB, b.wave_count, b.blk_ecount, b.num_tokens_per_rank,
                       b.num_tokens_per_expert, b.rank_prefix_matrix, b.channel_prefix_matrix,
                       b.recv_channel_prefix_matrix, b.num_recv);
    if (s.T > 0) {
        hipLaunchKernelGGL(layout_pos_kernel<NW>, dim3(s.nB), dim3(kLayoutBlock), 0, stream,
                           topk_idx, s.T, s.K, s.E, s.R, s.C, s.epr, s.kmax, s.nW, b.wave_mask,
                           b.wave_count, b.rank_prefix_matrix, b.is_token_in_rank, b.send_head,
                           b.recv_src_idx, b.dst_row, b.dst_rank, b.channel_prefix_matrix,
                           b.recv_channel_prefix_matrix);
    }
    return hipGetLastError();
}

}  // namespace

LayoutShape layout_shape(const ep_dims &d)
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
    s.nB = (s.T + kLayoutBlock - 1) / kLayoutBlock;
    return s;
}

size_t layout_arena_bytes(const LayoutShape &s, size_t off[14])
{
    const size_t T = size_t(s.T), R = size_t(s.R), E = size_t(s.E), C = size_t(s.C);
    const size_t km = size_t(s.kmax), nW = size_t(s.nW), nB = size_t(s.nB);
    const size_t sizes[14] = {
        R * 4,       E * 4,      T * R,       R * 4,       R * C * 4,   R * C * 4,  T * R * 4,
        T * km * 4,  T * km * 4, T * km * 4,  nW * R * 8,  R * nW * 4,  nB * E * 4, 8,
    };
    size_t cur = 0;
    for (int i = 0; i < 14; ++i) {
        off[i] = cur;
        cur += (sizes[i] + 255) & ~size_t(255);
    }
    return cur;
}

LayoutBufs layout_bufs_at(void *base, const size_t off[14])
{
    char *p = static_cast<char *>(base);
    LayoutBufs b;
    b.num_tokens_per_rank = reinterpret_cast<int32_t *>(p + off[0]);
    b.num_tokens_per_expert = reinterpret_cast<int32_t *>(p + off[1]);
    b.is_token_in_rank = reinterpret_cast<uint8_t *>(p + off[2]);
    b.rank_prefix_matrix = reinterpret_cast<int32_t *>(p + off[3]);
    b.channel_prefix_matrix = reinterpret_cast<int32_t *>(p + off[4]);
    b.recv_channel_prefix_matrix = reinterpret_cast<int32_t *>(p + off[5]);
    b.send_head = reinterpret_cast<int32_t *>(p + off[6]);
    b.recv_src_idx = reinterpret_cast<int32_t *>(p + off[7]);
    b.dst_row = reinterpret_cast<int32_t *>(p + off[8]);
    b.dst_rank = reinterpret_cast<int32_t *>(p + off[9]);
    b.wave_mask = reinterpret_cast<uint64_t *>(p + off[10]);
    b.wave_count = reinterpret_cast<int32_t *>(p + off[11]);
    b.blk_ecount = reinterpret_cast<int32_t *>(p + off[12]);
    b.num_recv = reinterpret_cast<int64_t *>(p + off[13]);
    return b;
}

hipError_t launch_layout(const LayoutShape &s, const int64_t *topk_idx, const LayoutBufs &b,
                         hipStream_t stream)
{
    switch ((s.R + kWave - 1) / kWave) {
    case 1: return launch_layout_nw<1>(s, topk_idx, b, stream);
    case 2: return launch_layout_nw<2>(s, topk_idx, b, stream);
    case 3: return launch_layout_nw<3>(s, topk_idx, b, stream);
    case 4: return launch_layout_nw<4>(s, topk_idx, b, stream);
    case 5:
    case 6: return launch_layout_nw<6>(s, topk_idx, b, stream);
    case 7:
    case 8: return launch_layout_nw<8>(s, topk_idx, b, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ep

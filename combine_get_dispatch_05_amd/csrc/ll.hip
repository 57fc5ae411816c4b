// ll.hip -- low-latency (decode) dispatch and combine on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "IB-GDA Kernels": low_latency_dispatch streams tokens straight into
// per-expert receive buffers with no intermediate staging and reports
// per-expert counts; low_latency_combine reduces the expert results back to
// the tokens' positions, weighted by the top-k weights.
//
// Dispatch is one fused launch with one workgroup per expert: the workgroup
// scans the [T][K] table, turns "names my expert" into slots with one
// block-wide prefix scan (so slots follow (token, slot) order), records the
// token of each slot, and then copies those token rows into the expert's
// area [le][r][slot][:] with every lane issuing independent 16-byte loads and
// stores.  No layout pass, no second launch, no host sync.
//
// Combine: one workgroup per (token, row chunk).  All K cell addresses of the
// token are resolved once into LDS; each lane then issues its K loads before
// the fused multiply-adds, which run in ascending slot order from +0.  A rank
// masked at combine time contributes nothing.
//
// FP8 ("use_fp8" of the same section, which the pages' code example sets on
// the dispatch): the dispatch can store e4m3 codes with one fp32 scale per
// 128 elements instead of bf16 rows.

#include <atomic>

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLLBlock = 256;
constexpr int kLLWaves = kLLBlock / kWave;

__device__ __forceinline__ int ll_wave_inclusive_scan(int v)
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

// OCP FP8 E4M3 ("e4m3fn") code of an fp32 value: round to nearest, ties to
// even, saturating at +-448 (no infinities in this format; 0x7F is NaN).
// Normal results: add just under half of the 20 dropped mantissa bits (plus
// one when the kept lsb is odd) and let a carry bump the exponent.  Results
// below 2^-6: scale by 2^9 (exact) and round to an integer count of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u)
        return sign | 0x7fu;
    if (a >= 0x43e00000u)  // 448.0f and above (infinity included)
        return sign | 0x7eu;
    if (a < 0x3c800000u)  // below 2^-6
        return sign | uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const uint32_t e = (r >> 23) - 127u + 7u;
    const uint32_t code = (e << 3) | ((r >> 20) & 7u);
    return sign | (code > 0x7eu ? 0x7eu : code);
}

// Max over each row of 16 lanes (the DPP row), every lane of the row gets
// the result: swaps within quads, then rotations by 4 and 8 inside the row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    uint32_t t = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false));
    v = v > t ? v : t;
    t = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false));
    v = v > t ? v : t;
    t = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x124, 0xF, 0xF, false));
    v = v > t ? v : t;
    t = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x128, 0xF, 0xF, false));
    return v > t ? v : t;
}

__device__ __forceinline__ float row16_fmax(float v)
{
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
        v = fmaxf(v, __shfl_xor(v, m, 16));
    return v;
}

// e4m3 codes of one 128-element block held by a 16-lane DPP row, 8 bf16 per
// lane (v), and the block's amax (after the 1e-4 floor).  Every lane of the
// row must take part.  Per block: amax = max(max |x|, 1e-4), code =
// e4m3(x * (448 / amax)) rounded to nearest even, saturating.
__device__ __forceinline__ uint2 fp8_block(const u32x4 &v, float &amax_out)
{
    // max |x| of the block as bf16 bits: for finite values the integer order
    // of the magnitude bits is the numeric order.
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = v[q];
        const uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
        bits = bits > lo ? bits : lo;
        bits = bits > hi ? bits : hi;
    }
    bits = row16_max(bits);
    uint2 codes;
    float amax;
    if (bits < 0x7f80u) {
        // finite block: |x * 448 / amax| stays below 464, where the hardware
        // conversion rounds to nearest even exactly as e4m3_rne does
        // (checked over every fp32 input).
        amax = __uint_as_float(bits << 16);
        amax = amax < 1e-4f ? 1e-4f : amax;
        const float sinv = 448.0f / amax;
        uint32_t c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t w0v = v[2 * h], w1v = v[2 * h + 1];
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w0v) * sinv, bf16_hi(w0v) * sinv, 0,
                                                     false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w1v) * sinv, bf16_hi(w1v) * sinv, pk,
                                                 true);
            c[h] = uint32_t(pk);
        }
        codes = make_uint2(c[0], c[1]);
    } else {
        // an infinity or NaN in the block: the general path
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = bf16_lo(v[q]);
            f[2 * q + 1] = bf16_hi(v[q]);
        }
        amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            amax = fmaxf(amax, fabsf(f[q]));
        amax = row16_fmax(amax);
        amax = amax < 1e-4f ? 1e-4f : amax;
        const float sinv = 448.0f / amax;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lo |= e4m3_rne(f[q] * sinv) << (8 * q);
            hi |= e4m3_rne(f[q + 4] * sinv) << (8 * q);
        }
        codes = make_uint2(lo, hi);
    }
    amax_out = amax;
    return codes;
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

// One workgroup per expert.  Each thread owns a contiguous chunk of the
// flattened [T][K] table (held in registers when it is short), counts the
// pairs naming its expert, and one block-wide exclusive scan of those counts
// gives every thread the first slot of its chunk, so slots follow (token,
// slot) order.  The rows are then copied with the (row, vector) pairs spread
// flat over the block, kUnroll independent 16-byte loads in flight per lane.
// A masked rank ("Dynamic Rank Masking") takes part in nothing: its experts'
// pairs get no slot and its counts are 0.
// kFP8: instead of bf16 rows, each 128-element block of a sent row is scaled
// by 448 / max(amax, 1e-4) and stored as e4m3 codes, with its scale
// amax / 448; a 16-lane group handles one block (8 elements per lane).
// The copy of one expert's rows is split over gridDim.y workgroups; each
// recomputes the (cheap, cached) slot scan, and only the y = 0 workgroup
// writes the metadata.
template <bool kFP8>
__global__ __launch_bounds__(kLLBlock) void ll_dispatch_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int R, int epr, int S,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask,
    u32x4 *__restrict__ packed_x, uint2 *__restrict__ packed_q, float *__restrict__ packed_scale,
    int32_t *__restrict__ packed_count, int32_t *__restrict__ src_info,
    int32_t *__restrict__ topk_slot)
{
    constexpr int kHold = 8;
    __shared__ int32_t s_tok[kMaxLLSlots];
    __shared__ int32_t s_wsum[kLLWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int e = blockIdx.x;
    const int le = e % epr;
    const int r = e / epr;
    const bool masked = rank_mask != nullptr && rank_mask[r] != 0;
    const int64_t cell0 = (int64_t(le) * R + r) * S;
    const int TK = T * K;
    const int chunk = (TK + kLLBlock - 1) / kLLBlock;
    const int i0 = tid * chunk;
    const int i1 = i0 + chunk < TK ? i0 + chunk : TK;
    const bool held = chunk <= kHold;

    int64_t v[kHold];
    int mine = 0;
    if (held) {
#pragma unroll
        for (int q = 0; q < kHold; ++q) {
            v[q] = i0 + q < i1 ? topk_idx[i0 + q] : -1;
            mine += (v[q] == e && !masked) ? 1 : 0;
        }
    } else {
        for (int i = i0; i < i1; ++i)
            mine += (topk_idx[i] == e && !masked) ? 1 : 0;
    }

    const int incl = ll_wave_inclusive_scan(mine);
    if (lane == kWave - 1)
        s_wsum[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kLLWaves; ++w) {
        const int c = s_wsum[w];
        before += w < wid ? c : 0;
        total += c;
    }
    int s = before + incl - mine;  // first slot of this thread's chunk

    const bool meta = blockIdx.y == 0;
    auto place = [&](int i, int64_t val) {
        if (val == e) {
            if (!masked && s < S) {
                if (meta) {
                    topk_slot[i] = s;
                    src_info[cell0 + s] = i / K;
                }
                s_tok[s] = i / K;
            } else if (meta) {
                topk_slot[i] = -1;
            }
            s += masked ? 0 : 1;
        } else if (meta && e == 0 && !(val >= 0 && val < E)) {
            topk_slot[i] = -1;  // masked or invalid slots: workgroup 0 marks them
        }
    };
    if (held) {
#pragma unroll
        for (int q = 0; q < kHold; ++q)
            if (i0 + q < i1)
                place(i0 + q, v[q]);
    } else {
        for (int i = i0; i < i1; ++i)
            place(i, topk_idx[i]);
    }

    const int used = total < S ? total : S;
    if (blockIdx.y == 0) {
        if (tid == 0)
            packed_count[int64_t(le) * R + r] = total;
        for (int q = used + tid; q < S; q += kLLBlock)
            src_info[cell0 + q] = -1;
    }
    __syncthreads();
    const int ny = gridDim.y, yb = blockIdx.y;

    if (!kFP8 && packed_x != nullptr) {
        constexpr int kUnroll = 8;
        const int n = used * V;
        for (int p0 = yb * kLLBlock * kUnroll; p0 < n; p0 += ny * kLLBlock * kUnroll) {
            u32x4 buf[kUnroll];
            int64_t dst[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int p = p0 + u * kLLBlock + tid;
                dst[u] = -1;
                if (p < n) {
                    const int row = p / V;
                    const int col = p - row * V;
                    buf[u] = x[int64_t(s_tok[row]) * V + col];
                    dst[u] = (cell0 + row) * V + col;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (dst[u] >= 0)
                    packed_x[dst[u]] = buf[u];
        }
    }

    if (kFP8) {
        // 16 vectors of 8 bf16 per 128-element block; V is a multiple of 16.
        // A wave takes 4 blocks per round and kRounds rounds at once, so
        // kRounds loads are in flight before any block is quantized.  Lanes
        // past the end load row 0's block (always valid when items > 0) and
        // store nothing.
        constexpr int kRounds = 4;
        const int nb = V / 16;
        const int items = used * nb;
        const int g16 = lane >> 4;  // group of 16 lanes inside the wave
        const int l16 = lane & 15;
        const int wave = yb * kLLWaves + wid;
        const int nwaves = ny * kLLWaves;
        for (int w0 = wave * 4 * kRounds; w0 < items; w0 += nwaves * 4 * kRounds) {
            u32x4 vv[kRounds];
            int row[kRounds], blk[kRounds], tok[kRounds];
#pragma unroll
            for (int k = 0; k < kRounds; ++k) {
                const int item = w0 + k * 4 + g16;
                const int it = item < items ? item : 0;
                row[k] = item < items ? it / nb : -1;
                blk[k] = it - (it / nb) * nb;
                tok[k] = s_tok[it / nb];
            }
#pragma unroll
            for (int k = 0; k < kRounds; ++k)
                vv[k] = x[int64_t(tok[k]) * V + int64_t(blk[k]) * 16 + l16];
#pragma unroll
            for (int k = 0; k < kRounds; ++k) {
                float amax;
                const uint2 codes = fp8_block(vv[k], amax);
                if (row[k] >= 0) {
                    const int64_t cell = cell0 + row[k];
                    const int64_t col = int64_t(blk[k]) * 16 + l16;
                    packed_q[cell * V + col] = codes;  // 8 codes per lane
                    if (l16 == 0)
                        packed_scale[cell * nb + blk[k]] = amax / 448.0f;
                }
            }
        }
    }
}

constexpr int kLLTokPairs = 4096;  // token-major path for T*K up to this (ids held in LDS)
constexpr int kSlotChunk = 8;      // a token's experts matched per pass of the slot scan

// Token-major variant for small batches (T*K <= kLLTokPairs), same results
// as ll_dispatch_kernel.  Every workgroup first loads the whole [T][K] id
// table into LDS.  Workgroups [0, T*ny) are token workgroups: (t, slice y).
// The slot of an own pair (t, k) is the number of earlier pairs (in (token,
// slot) order) that name the same expert: all lanes of the workgroup scan the
// earlier tokens' pairs once, each entry compared with up to kSlotChunk of
// the token's experts, the per-lane counts are added up in LDS, and thread k
// adds the token's own earlier slots.  The slice of x[t] is then read once
// and stored to all K destination cells (for FP8 each 128-element block is
// quantized once).  The remaining workgroups handle four experts each (one
// per wave): the expert's count and the -1 entries of its unused src_info
// cells.
template <bool kFP8>
__global__ __launch_bounds__(kLLBlock) void ll_dispatch_tok_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int R, int epr, int S, int ny,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask,
    u32x4 *__restrict__ packed_x, uint2 *__restrict__ packed_q, float *__restrict__ packed_scale,
    int32_t *__restrict__ packed_count, int32_t *__restrict__ src_info,
    int32_t *__restrict__ topk_slot)
{
    __shared__ int32_t s_ids[kLLTokPairs];
    __shared__ int64_t s_cell[kMaxTopk];
    __shared__ int32_t s_cnt[kMaxTopk];  // earlier tokens' pairs naming pair k's expert
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int TK = T * K;
    const int b = blockIdx.x;
    const int ntok = T * ny;
    const int t = b / ny;
    const int yb = b - t * ny;

    // The first vector of this lane's share of the row slice does not depend
    // on the slots: its load is issued before anything else.
    int c0 = 0, c1 = 0, b0 = 0, b1 = 0;
    u32x4 first = {0, 0, 0, 0};
    if (b < ntok) {
        if (!kFP8) {
            const int per = (V + ny - 1) / ny;
            c0 = yb * per;
            c1 = c0 + per < V ? c0 + per : V;
            if (packed_x != nullptr && c0 + tid < c1)
                first = x[int64_t(t) * V + c0 + tid];
        } else {
            const int nb = V / 16;
            const int per = (nb + ny - 1) / ny;
            b0 = yb * per;
            b1 = b0 + per < nb ? b0 + per : nb;
            if (b0 + (tid >> 4) < b1)
                first = x[int64_t(t) * V + int64_t(b0 + (tid >> 4)) * 16 + (tid & 15)];
        }
    }

    if (tid < kMaxTopk)
        s_cnt[tid] = 0;
    // expert id of every pair; -1 for masked slots and invalid ids
    constexpr int kU = 4;
    for (int i0 = 0; i0 < TK; i0 += kLLBlock * kU) {
        int64_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kLLBlock + tid;
            v[u] = i < TK ? topk_idx[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = i0 + u * kLLBlock + tid;
            if (i < TK)
                s_ids[i] = (v[u] >= 0 && v[u] < E) ? int(v[u]) : -1;
        }
    }
    __syncthreads();

    if (b >= ntok) {
        const int e = (b - ntok) * kLLWaves + wid;
        if (e < E) {
            const int r = e / epr;
            const bool masked = rank_mask != nullptr && rank_mask[r] != 0;
            int cnt = 0;
            if (!masked)
                for (int i = lane; i < TK; i += kWave)
                    cnt += s_ids[i] == e ? 1 : 0;
            cnt = wave_sum(cnt);
            const int64_t cell0 = (int64_t(e - r * epr) * R + r) * S;
            if (lane == 0)
                packed_count[int64_t(e - r * epr) * R + r] = cnt;
            for (int q = (cnt < S ? cnt : S) + lane; q < S; q += kWave)
                src_info[cell0 + q] = -1;
        }
        return;
    }

    // Thread k < K owns pair (t, k); its rank-mask load is issued before the
    // scan so that the scan hides its latency.
    const int base = t * K;
    int e_mine = -1;
    bool live_mine = false;
    if (tid < K) {
        e_mine = s_ids[base + tid];
        live_mine = e_mine >= 0 && (rank_mask == nullptr || rank_mask[e_mine / epr] == 0);
    }
    // An expert occurs only a few times among the earlier pairs, so the few
    // nonzero per-lane counts go to LDS with atomic adds.
    for (int k0 = 0; k0 < K; k0 += kSlotChunk) {
        int ek[kSlotChunk], c[kSlotChunk];
#pragma unroll
        for (int q = 0; q < kSlotChunk; ++q) {
            ek[q] = k0 + q < K ? s_ids[base + k0 + q] : -2;  // -2 matches no entry
            c[q] = 0;
        }
        for (int i = tid; i < base; i += kLLBlock) {
            const int v = s_ids[i];
#pragma unroll
            for (int q = 0; q < kSlotChunk; ++q)
                c[q] += v == ek[q] ? 1 : 0;
        }
#pragma unroll
        for (int q = 0; q < kSlotChunk; ++q)
            if (c[q] != 0)
                atomicAdd(&s_cnt[k0 + q], c[q]);
    }
    __syncthreads();
    if (tid < K) {
        int64_t cell = -1;
        int slot = -1;
        if (live_mine) {
            int cnt = s_cnt[tid];
            for (int j = 0; j < tid; ++j)
                cnt += s_ids[base + j] == e_mine ? 1 : 0;
            if (cnt < S) {
                const int r = e_mine / epr;
                slot = cnt;
                cell = (int64_t(e_mine - r * epr) * R + r) * S + cnt;
            }
        }
        s_cell[tid] = cell;
        if (yb == 0) {
            topk_slot[base + tid] = slot;
            if (cell >= 0)
                src_info[cell] = t;
        }
    }
    __syncthreads();  // s_cell is read by the copy below

    if (!kFP8) {
        if (packed_x == nullptr)
            return;
        for (int c = c0 + tid; c < c1; c += kLLBlock) {
            const u32x4 v = c == c0 + tid ? first : x[int64_t(t) * V + c];
            for (int k = 0; k < K; ++k) {
                const int64_t cell = s_cell[k];
                if (cell >= 0)
                    packed_x[cell * V + c] = v;
            }
        }
    } else {
        // 16 lane groups, one 128-element block each; a group is a DPP row,
        // and a block's loop bounds are the same for all of its lanes.
        const int nb = V / 16;
        const int g = tid >> 4;
        const int l16 = tid & 15;
        for (int bb = b0 + g; bb < b1; bb += kLLBlock / 16) {
            const u32x4 v = bb == b0 + g ? first : x[int64_t(t) * V + int64_t(bb) * 16 + l16];
            float amax;
            const uint2 codes = fp8_block(v, amax);
            for (int k = 0; k < K; ++k) {
                const int64_t cell = s_cell[k];
                if (cell >= 0) {
                    packed_q[cell * V + int64_t(bb) * 16 + l16] = codes;
                    if (l16 == 0)
                        packed_scale[cell * nb + bb] = amax / 448.0f;
                }
            }
        }
    }
}

template <int VPT>
__global__ __launch_bounds__(kLLBlock) void ll_combine_kernel(
    const u32x4 *__restrict__ packed_y, int V, int K, int E, int R, int epr, int S,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    const int32_t *__restrict__ topk_slot, const int32_t *__restrict__ rank_mask,
    u32x4 *__restrict__ out)
{
    __shared__ int64_t s_cell[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    if (tid < K) {
        const int64_t e = topk_idx[t * K + tid];
        const int s = topk_slot[t * K + tid];
        const bool ok = e >= 0 && e < E && s >= 0 && s < S &&
                        !(rank_mask != nullptr && rank_mask[int(e) / epr] != 0);
        s_cell[tid] = ok ? ((int64_t(int(e) % epr) * R + int(e) / epr) * S + s) : -1;
        s_w[tid] = topk_weights[t * K + tid];
    }
    __syncthreads();

    const int base = blockIdx.y * kLLBlock * VPT;
    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = 0.0f;

    constexpr int kGroup = 8;
    for (int k0 = 0; k0 < K; k0 += kGroup) {
        u32x4 v[kGroup][VPT];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            const int64_t cell = k < K ? s_cell[k] : -1;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kLLBlock + tid;
                v[g][i] = (cell >= 0 && idx < V) ? packed_y[cell * V + idx] : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            if (k < K && s_cell[k] >= 0) {
                const float w = s_w[k];
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[i][2 * q] = __builtin_fmaf(w, bf16_lo(v[g][i][q]), acc[i][2 * q]);
                        acc[i][2 * q + 1] =
                            __builtin_fmaf(w, bf16_hi(v[g][i][q]), acc[i][2 * q + 1]);
                    }
                }
            }
        }
    }

    u32x4 *o = out + t * V;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int idx = base + i * kLLBlock + tid;
        if (idx < V) {
            u32x4 rv;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rv[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
            o[idx] = rv;
        }
    }
}

// The combine of an FP8 payload (codes and per-128-element-block scales, as
// the FP8 dispatch stores them).  A lane takes 8 elements of the row (one
// 8-byte word of codes per cell); each code is decoded exactly with the
// packed hardware conversion (checked against the e4m3 definition for all
// 256 codes), multiplied by its block's scale in fp32, and added with the
// same fma sum in ascending k as the bf16 combine.
__global__ __launch_bounds__(kLLBlock) void ll_combine_fp8_kernel(
    const uint2 *__restrict__ packed_q, const float *__restrict__ packed_scale, int V, int K,
    int E, int R, int epr, int S, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ topk_slot,
    const int32_t *__restrict__ rank_mask, u32x4 *__restrict__ out)
{
    __shared__ int64_t s_cell[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    if (tid < K) {
        const int64_t e = topk_idx[t * K + tid];
        const int s = topk_slot[t * K + tid];
        const bool ok = e >= 0 && e < E && s >= 0 && s < S &&
                        !(rank_mask != nullptr && rank_mask[int(e) / epr] != 0);
        s_cell[tid] = ok ? ((int64_t(int(e) % epr) * R + int(e) / epr) * S + s) : -1;
        s_w[tid] = topk_weights[t * K + tid];
    }
    __syncthreads();

    const int idx = blockIdx.y * kLLBlock + tid;  // 8-element group of the row
    const int nb = V / 16;                          // 128-element blocks per row
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = 0.0f;

    constexpr int kGroup = 8;
    for (int k0 = 0; k0 < K; k0 += kGroup) {
        uint2 c[kGroup];
        float sc[kGroup];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            const int64_t cell = k < K ? s_cell[k] : -1;
            const bool live = cell >= 0 && idx < V;
            c[g] = live ? packed_q[cell * V + idx] : make_uint2(0, 0);
            sc[g] = live ? packed_scale[cell * nb + idx / 16] : 0.0f;
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            if (k < K && s_cell[k] >= 0) {
                const float w = s_w[k];
                const uint32_t words[2] = {c[g].x, c[g].y};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(words[h]), false);
                    const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(words[h]), true);
                    acc[4 * h + 0] = __builtin_fmaf(w, d01[0] * sc[g], acc[4 * h + 0]);
                    acc[4 * h + 1] = __builtin_fmaf(w, d01[1] * sc[g], acc[4 * h + 1]);
                    acc[4 * h + 2] = __builtin_fmaf(w, d23[0] * sc[g], acc[4 * h + 2]);
                    acc[4 * h + 3] = __builtin_fmaf(w, d23[1] * sc[g], acc[4 * h + 3]);
                }
            }
        }
    }
    if (idx < V) {
        u32x4 rv;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            rv[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        out[t * V + idx] = rv;
    }
}

std::atomic<int> g_ll_mode{0};  // 0 automatic, 1 expert-major, 2 token-major when it fits

}  // namespace

bool set_ll_tuning(int mode)
{
    if (mode < 0 || mode > 2)
        return false;
    g_ll_mode = mode;
    return true;
}

hipError_t launch_ll_dispatch(const ep_dims &d, int num_slots, const void *x,
                              const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                              void *packed_q, float *packed_scale, int32_t *packed_count,
                              int32_t *src_info, int32_t *topk_slot, hipStream_t stream)
{
    const int E = d.num_experts, R = d.num_ranks;
    const bool fp8 = packed_q != nullptr;
    const int64_t TK = int64_t(d.num_tokens) * d.num_topk;
    if (g_ll_mode.load() != 1 && TK <= kLLTokPairs) {
        // token-major: slices of about 256 vectors (bf16) or 16 blocks (fp8)
        const int V = d.hidden / 8;
        const bool rows = fp8 || packed_x != nullptr;
        int ny = 1;
        if (rows)
            ny = fp8 ? (V / 16 + 15) / 16 : (V + kLLBlock - 1) / kLLBlock;
        const int64_t blocks = int64_t(d.num_tokens) * ny + (E + kLLWaves - 1) / kLLWaves;
        if (log_enabled())
            log_launch("ll_dispatch token-major T=%d H=%d K=%d E=%d: slices=%d blocks=%lld%s",
                       d.num_tokens, d.hidden, d.num_topk, E, ny, (long long)blocks,
                       fp8 ? " fp8" : "");
        auto tk = fp8 ? ll_dispatch_tok_kernel<true> : ll_dispatch_tok_kernel<false>;
        hipLaunchKernelGGL(tk, dim3(unsigned(blocks)), dim3(kLLBlock), 0, stream,
                           static_cast<const u32x4 *>(x), d.num_tokens, V, d.num_topk, E, R,
                           E / R, num_slots, ny, topk_idx, rank_mask,
                           static_cast<u32x4 *>(packed_x), static_cast<uint2 *>(packed_q),
                           packed_scale, packed_count, src_info, topk_slot);
        return hipGetLastError();
    }
    auto kernel = fp8 ? ll_dispatch_kernel<true> : ll_dispatch_kernel<false>;
    // Copy splits per expert, from the expected rows per expert T*K/E: one
    // workgroup round copies 2048 vectors (bf16) or 64 blocks (fp8).
    const int64_t rows = (int64_t(d.num_tokens) * d.num_topk + E - 1) / E;
    const int64_t work = fp8 ? rows * (d.hidden / 128) : rows * (d.hidden / 8);
    const int64_t per = fp8 ? 64 : 2048;
    int ny = int((work + per - 1) / per);
    ny = ny < 1 ? 1 : (ny > 8 ? 8 : ny);
    if (log_enabled())
        log_launch("ll_dispatch expert-major T=%d H=%d K=%d E=%d: grid=%dx%d%s", d.num_tokens,
                   d.hidden, d.num_topk, E, E, ny, fp8 ? " fp8" : "");
    hipLaunchKernelGGL(kernel, dim3(E, ny), dim3(kLLBlock), 0, stream,
                       static_cast<const u32x4 *>(x), d.num_tokens, d.hidden / 8, d.num_topk, E,
                       R, E / R, num_slots, topk_idx, rank_mask, static_cast<u32x4 *>(packed_x),
                       static_cast<uint2 *>(packed_q), packed_scale, packed_count, src_info,
                       topk_slot);
    return hipGetLastError();
}

hipError_t launch_ll_combine_fp8(const ep_dims &d, int num_slots, const void *packed_q,
                                 const float *packed_scale, const int64_t *topk_idx,
                                 const float *topk_weights, const int32_t *topk_slot,
                                 const int32_t *rank_mask, void *out, hipStream_t stream)
{
    if (d.num_tokens == 0)
        return hipSuccess;
    const int E = d.num_experts, R = d.num_ranks;
    const int V = d.hidden / 8;
    const int chunks = (V + kLLBlock - 1) / kLLBlock;
    if (log_enabled())
        log_launch("ll_combine fp8 T=%d H=%d K=%d: grid=%dx%d", d.num_tokens, d.hidden,
                   d.num_topk, d.num_tokens, chunks);
    hipLaunchKernelGGL(ll_combine_fp8_kernel, dim3(d.num_tokens, chunks), dim3(kLLBlock), 0,
                       stream, static_cast<const uint2 *>(packed_q), packed_scale, V, d.num_topk,
                       E, R, E / R, num_slots, topk_idx, topk_weights, topk_slot, rank_mask,
                       static_cast<u32x4 *>(out));
    return hipGetLastError();
}

hipError_t launch_ll_combine(const ep_dims &d, int num_slots, const void *packed_y,
                             const int64_t *topk_idx, const float *topk_weights,
                             const int32_t *topk_slot, const int32_t *rank_mask, void *out,
                             hipStream_t stream)
{
    if (d.num_tokens == 0)
        return hipSuccess;
    const int E = d.num_experts, R = d.num_ranks;
    const int V = d.hidden / 8;
    constexpr int VPT = 1;
    const int chunks = (V + kLLBlock * VPT - 1) / (kLLBlock * VPT);
    if (log_enabled())
        log_launch("ll_combine T=%d H=%d K=%d: grid=%dx%d", d.num_tokens, d.hidden, d.num_topk,
                   d.num_tokens, chunks);
    hipLaunchKernelGGL((ll_combine_kernel<VPT>), dim3(d.num_tokens, chunks), dim3(kLLBlock), 0,
                       stream, static_cast<const u32x4 *>(packed_y), V, d.num_topk, E, R, E / R,
                       num_slots, topk_idx, topk_weights, topk_slot, rank_mask,
                       static_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace ep

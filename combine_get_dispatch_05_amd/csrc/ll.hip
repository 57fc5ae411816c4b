// ll.hip -- low-latency (decode) dispatch and combine on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "IB-GDA Kernels": low_latency_dispatch streams tokens straight into
// per-expert receive buffers with no intermediate staging and reports
// per-expert counts; low_latency_combine reduces the expert results back to
// the tokens' positions, weighted by the top-k weights.
//
// Dispatch of a decode-sized batch (T*K <= 4096) is one launch: each
// workgroup owns one slice of one token's row, finds the slots of the
// token's K pairs (the number of earlier pairs naming the same expert) with
// wave ballots over top-k ids held in registers, and stores the slice, read
// once, to the K destination cells [le][r][slot][:].  Larger batches take
// two launches: a per-expert slot scan, then the same token-major copy.  No
// layout pass and no host sync either way.
//
// Combine: one workgroup per (token, row chunk).  Every wave resolves the
// token's K cell addresses in its first K lanes; each lane then issues its K loads before
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

// Threads of a workgroup that moves one row slice: the dispatch's token
// workgroups, the copy and both combines.  All of them cut a row into the
// same slices and number their workgroups (token, slice) in the same order.
// Workgroup i runs on XCD i mod 8, so the combine reads each cell line on
// the XCD whose L2 wrote it in the dispatch.
constexpr int kTokBlock = 512;

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
        // conversion rounds to nearest even, saturating, as the e4m3
        // definition does (test_ll_dispatch_fp8_conversion_sweep compares
        // the codes bit for bit on every bf16 magnitude up to the block's
        // amax, for a scale of exactly 1 and for scales that are not powers
        // of two).
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

// Expert id of one top-k entry: -1 for a masked slot or an id outside [0, E).
__device__ __forceinline__ int ll_valid_id(int64_t v, int E)
{
    return (v >= 0 && v < E) ? int(v) : -1;
}

// Rank of expert e >= 0 (epr experts per rank): a shift when epr is a power
// of two (a uniform test), else a division.
__device__ __forceinline__ int ll_rank(int e, int epr)
{
    if ((epr & (epr - 1)) == 0)
        return e >> __builtin_ctz(unsigned(epr));
    return e / epr;
}

// Index of cell (le, r, s) of expert e in the [E/R][R][S] receive layout.
// E * S <= 8192 * 4096, so it fits an int.
__device__ __forceinline__ int ll_cell(int e, int epr, int R, int S, int s)
{
    const int r = ll_rank(e, epr);
    return ((e - r * epr) * R + r) * S + s;
}

__device__ __forceinline__ int ll_readlane(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

// Packed rows are read again soon (by the expert computation and the
// combine): plain stores leave them in the caches.  Nontemporal stores made
// the dispatch 0.3 us faster and the combine after it 2.4 us slower.
__device__ __forceinline__ void ll_store(u32x4 v, u32x4 *p) { *p = v; }

// This workgroup's slice of token t's row, stored to the cells of the
// token's K pairs (lane k of every wave holds pair k's cell, -1 for none).
// bf16: vectors [c0, c1) of the row, the lane's first one already loaded
// in `first`.  FP8: 128-element blocks [b0, b1), one per 16-lane group (a
// DPP row, so a block's loop bounds are the same for all of its lanes),
// each quantized once and stored K times.
template <bool kFP8, int BT>
__device__ __forceinline__ void ll_store_slice(const u32x4 *__restrict__ x, int64_t t, int V,
                                               int K, int cell, u32x4 first, int c0, int c1,
                                               int b0, int b1, u32x4 *__restrict__ packed_x,
                                               uint2 *__restrict__ packed_q,
                                               float *__restrict__ packed_scale)
{
    const int tid = threadIdx.x;
    if (!kFP8) {
        for (int c = c0 + tid; c < c1; c += BT) {
            const u32x4 v = c == c0 + tid ? first : x[t * V + c];
            for (int k = 0; k < K; ++k) {
                const int ck = ll_readlane(cell, k);
                if (ck >= 0)
                    ll_store(v, packed_x + int64_t(ck) * V + c);
            }
        }
    } else {
        const int nb = V / 16;
        const int g = tid >> 4;
        const int l16 = tid & 15;
        for (int bb = b0 + g; bb < b1; bb += BT / 16) {
            const u32x4 v = bb == b0 + g ? first : x[t * V + int64_t(bb) * 16 + l16];
            float amax;
            const uint2 codes = fp8_block(v, amax);
            for (int k = 0; k < K; ++k) {
                const int ck = ll_readlane(cell, k);
                if (ck >= 0) {
                    packed_q[int64_t(ck) * V + int64_t(bb) * 16 + l16] = codes;
                    if (l16 == 0)
                        packed_scale[int64_t(ck) * nb + bb] = amax / 448.0f;
                }
            }
        }
    }
}

// Row slice of workgroup `yb` of ny: vectors [c0, c1) (bf16, about 256
// vectors) or 128-element blocks [b0, b1) (FP8, about 16 blocks).
template <bool kFP8>
__device__ __forceinline__ void ll_slice(int V, int ny, int yb, int &c0, int &c1, int &b0, int &b1)
{
    if (!kFP8) {
        const int per = (V + ny - 1) / ny;
        c0 = yb * per;
        c1 = c0 + per < V ? c0 + per : V;
        b0 = b1 = 0;
    } else {
        const int nb = V / 16;
        const int per = (nb + ny - 1) / ny;
        b0 = yb * per;
        b1 = b0 + per < nb ? b0 + per : nb;
        c0 = c1 = 0;
    }
}

// The first vector of this lane's share of the slice (its load does not
// depend on the slots, so it is issued before they are known).  A slice is
// never empty (checked for every row length and block size the library
// accepts), and lanes past its end read its last vector again (never
// stored), so the load is unconditional: no per-lane branch makes later
// waits conservative.  kRows = false (metadata only): no load at all.
template <bool kFP8, bool kRows>
__device__ __forceinline__ u32x4 ll_first(const u32x4 *__restrict__ x, int64_t t, int V, int c0,
                                          int c1, int b0, int b1)
{
    const int tid = threadIdx.x;
    u32x4 v = {0, 0, 0, 0};
    if (!kRows)
        return v;
    if (!kFP8) {
        const int c = c0 + tid;
        v = x[t * V + (c < c1 ? c : c1 - 1)];
    } else {
        const int bb = b0 + (tid >> 4);
        v = x[t * V + int64_t(bb < b1 ? bb : b1 - 1) * 16 + (tid & 15)];
    }
    return v;
}

// Slot scan for batches of any size, one workgroup per expert.  The
// flattened [T][K] table is read in rounds of kHold * kSlotBlock entries
// (kHold picked per launch from the table size), coalesced: entry
// j * kSlotBlock + tid of the round goes to thread tid, so the
// round's entries in index order are ordered by (j, wave, lane).  Each wave
// takes one ballot per j of the entries naming the workgroup's expert; the
// per-(j, wave) counts go to LDS and, behind one barrier, every wave scans
// them (two per lane), so a matching lane's slot is the matches before its
// row and wave plus a popcount of the ballot below its lane: slots follow
// (token, slot) order.  Writes the expert's count, src_info (-1 in unused
// cells) and topk_slot of its pairs; workgroup 0 also marks masked and
// invalid slots.  A masked rank ("Dynamic Rank Masking") takes part in
// nothing: its experts' pairs get no slot and its counts are 0.  The rows
// are copied afterwards by ll_copy_kernel, token-major, so each token row is
// read once.
constexpr int kSlotBlock = 512;
constexpr int kSlotWaves = kSlotBlock / kWave;
constexpr int kSlotMaxHold = 16;  // table entries per thread and round, at most

template <int kHold>
__global__ __launch_bounds__(kSlotBlock) void ll_slot_kernel(
    int T, int K, int E, int R, int epr, int S, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ rank_mask, int32_t *__restrict__ packed_count,
    int32_t *__restrict__ src_info, int32_t *__restrict__ topk_slot)
{
    constexpr int kRound = kSlotBlock * kHold;
    constexpr int kCounts = kHold * kSlotWaves;
    static_assert(kCounts <= 2 * kWave, "at most two (row, wave) counts per lane");
    // counts of (row j, wave w) at j * kSlotWaves + w; two buffers, so that a
    // round's writes never meet the previous round's reads
    __shared__ int32_t s_cnt[2][kCounts];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = blockIdx.x;
    const int le = e % epr;
    const int r = e / epr;
    const bool masked = rank_mask != nullptr && rank_mask[r] != 0;
    const int cell0 = (le * R + r) * S;
    const int TK = T * K;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int carry = 0;  // matches in earlier rounds

    for (int base = 0, round = 0; base < TK; base += kRound, ++round) {
        // every load in flight (indexes clamped into the table) before any test
        int64_t raw[kHold];
#pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const int i = base + j * kSlotBlock + tid;
            raw[j] = topk_idx[i < TK ? i : TK - 1];
        }
        int32_t *cnt = s_cnt[round & 1];
        uint64_t m[kHold];
#pragma unroll
        for (int j = 0; j < kHold; ++j) {
            const int i = base + j * kSlotBlock + tid;
            m[j] = __builtin_amdgcn_ballot_w64(i < TK && raw[j] == e);
            if (lane == 0)
                cnt[j * kSlotWaves + wid] = __popcll(m[j]);
        }
        __syncthreads();
        // exclusive scan of the round's counts in (j, wave) order: lane l
        // holds positions l and l + 64 (0 past the end)
        const int c_lo = lane < kCounts ? cnt[lane] : 0;
        const int c_hi = lane + kWave < kCounts ? cnt[lane + kWave] : 0;
        int s_lo = c_lo, s_hi = c_hi;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int n_lo = __shfl_up(s_lo, o, kWave);
            const int n_hi = __shfl_up(s_hi, o, kWave);
            if (lane >= o) {
                s_lo += n_lo;
                s_hi += n_hi;
            }
        }
        const int tot_lo = __builtin_amdgcn_readlane(s_lo, kWave - 1);
        const int ex_lo = carry + s_lo - c_lo;
        const int ex_hi = carry + tot_lo + s_hi - c_hi;
#pragma unroll
        for (int j = 0; j < kHold; ++j) {
            if (m[j] == 0)
                continue;
            const int idx = j * kSlotWaves + wid;
            const int pre = idx < kWave ? __builtin_amdgcn_readlane(ex_lo, idx)
                                        : __builtin_amdgcn_readlane(ex_hi, idx - kWave);
            if ((m[j] >> lane) & 1) {
                const int i = base + j * kSlotBlock + tid;
                const int s = pre + __popcll(m[j] & below);
                if (!masked && s < S) {
                    topk_slot[i] = s;
                    src_info[cell0 + s] = i / K;
                } else {
                    topk_slot[i] = -1;
                }
            }
        }
        if (e == 0) {
            // masked or invalid slots: workgroup 0 marks them
#pragma unroll
            for (int j = 0; j < kHold; ++j) {
                const int i = base + j * kSlotBlock + tid;
                if (i < TK && ll_valid_id(raw[j], E) < 0)
                    topk_slot[i] = -1;
            }
        }
        carry += tot_lo + __builtin_amdgcn_readlane(s_hi, kWave - 1);
    }

    const int total = masked ? 0 : carry;
    const int used = total < S ? total : S;
    if (tid == 0)
        packed_count[le * R + r] = total;
    for (int q = used + tid; q < S; q += kSlotBlock)
        src_info[cell0 + q] = -1;
}

// Row copy after ll_slot_kernel, token-major: workgroup (t, slice) reads its
// slice of x[t] once and stores it to the cells of the token's pairs, which
// come from topk_slot.
template <bool kFP8>
__global__ __launch_bounds__(kTokBlock) void ll_copy_kernel(
    const u32x4 *__restrict__ x, int V, int K, int E, int R, int epr, int S, int ny,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ topk_slot,
    u32x4 *__restrict__ packed_x, uint2 *__restrict__ packed_q, float *__restrict__ packed_scale)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = blockIdx.x / ny;
    const int yb = blockIdx.x - int(t) * ny;
    int c0, c1, b0, b1;
    ll_slice<kFP8>(V, ny, yb, c0, c1, b0, b1);
    // the pair's id and slot (lanes past K read pair K - 1 again) and the
    // slice's first vector, all in flight before any is looked at
    const int k = lane < K ? lane : K - 1;
    int64_t e_raw = topk_idx[t * K + k];
    int s = topk_slot[t * K + k];
    const u32x4 first = ll_first<kFP8, true>(x, t, V, c0, c1, b0, b1);
    asm volatile("" : "+v"(e_raw), "+v"(s));
    const int e = ll_valid_id(e_raw, E);
    const int cell = (lane < K && e >= 0 && s >= 0 && s < S) ? ll_cell(e, epr, R, S, s) : -1;
    ll_store_slice<kFP8, kTokBlock>(x, t, V, K, cell, first, c0, c1, b0, b1, packed_x, packed_q,
                                   packed_scale);
}

constexpr int kLLTokPairs = 4096;  // one-launch path for T*K up to this

// Wave-wide count of the lanes where p holds.
__device__ __forceinline__ int ll_count(bool p)
{
    return __popcll(__builtin_amdgcn_ballot_w64(p));
}

// One-launch dispatch for decode-sized batches (T*K <= kLLTokPairs), same
// results as ll_slot_kernel + ll_copy_kernel.  Workgroups [0, T*ny) are
// token workgroups (t, slice).  The slot of pair (t, k) is the number of
// earlier pairs, in (token, slot) order, that name its expert: those of
// earlier tokens, plus the token's own pairs before k.  Every thread holds
// kRegs entries of the table in registers (coalesced loads, entries of
// token t and later replaced by -1); for each k, one ballot per register
// counts the wave's matches, and lane k keeps the count.  The waves' counts
// meet in LDS behind the one barrier.  The token's own earlier pairs are one
// more ballot over the lanes holding its ids.  The slice of x[t] (its first
// load issued before any id is looked at) is then stored to all K cells; for
// FP8 each 128-element block is quantized once.  The remaining workgroups
// handle BT/64 experts each (one per wave), counting with the same ballots
// over the whole table: the expert's count and the -1 entries of its unused
// src_info cells.
template <bool kFP8, int BT, bool kRows, int kRegs>
__global__ __launch_bounds__(BT) void ll_dispatch_tok_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int R, int epr, int S, int ny,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ rank_mask,
    u32x4 *__restrict__ packed_x, uint2 *__restrict__ packed_q, float *__restrict__ packed_scale,
    int32_t *__restrict__ packed_count, int32_t *__restrict__ src_info,
    int32_t *__restrict__ topk_slot)
{
    constexpr int kWaves = BT / kWave;
    __shared__ int32_t s_part[kMaxTopk][kWaves];  // per-wave match counts
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int TK = T * K;
    const int b = blockIdx.x;
    const int ntok = T * ny;

    if (b >= ntok) {
        // experts e0 .. e0 + kWaves - 1, one per wave: matches over the whole
        // table (positions past its end hold -1)
        const int e0 = (b - ntok) * kWaves;
        int64_t raw[kRegs];
#pragma unroll
        for (int u = 0; u < kRegs; ++u)
            raw[u] = -1;
        if (TK > 0) {  // T = 0: the counts are 0 and every cell unused
#pragma unroll
            for (int u = 0; u < kRegs; ++u) {
                const int i = u * BT + tid;
                raw[u] = topk_idx[i < TK ? i : TK - 1];
            }
        }
        int ids[kRegs];
#pragma unroll
        for (int u = 0; u < kRegs; ++u)
            ids[u] = u * BT + tid < TK ? ll_valid_id(raw[u], E) : -1;
        int mine = 0;  // lane j: the count of expert e0 + j
#pragma unroll
        for (int j = 0; j < kWaves; ++j) {
            int c = 0;
#pragma unroll
            for (int u = 0; u < kRegs; ++u)
                c += ll_count(ids[u] == e0 + j);
            mine = lane == j ? c : mine;
        }
        if (lane < kWaves)
            s_part[lane][wid] = mine;
        __syncthreads();
        const int e = e0 + wid;
        if (e < E) {
            const int r = e / epr;
            const bool masked = rank_mask != nullptr && rank_mask[r] != 0;
            int cnt = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                cnt += s_part[wid][w];
            cnt = masked ? 0 : cnt;
            const int cell0 = ll_cell(e, epr, R, S, 0);
            if (lane == 0)
                packed_count[(e - r * epr) * R + r] = cnt;
            for (int q = (cnt < S ? cnt : S) + lane; q < S; q += kWave)
                src_info[cell0 + q] = -1;
        }
        return;
    }

    const int t = b / ny;
    const int yb = b - t * ny;
    const int base = t * K;  // pairs of earlier tokens
    // Loads first, all in flight at once: lane k < K's own pair (t, k)
    // (lanes past K read pair K - 1 again), the table entries of earlier
    // tokens (indexes clamped; entries from position base on are replaced
    // by -1 below), then the row slice's first vector.
    int64_t own_raw = topk_idx[base + (lane < K ? lane : K - 1)];
    const int last = base > 0 ? base - 1 : 0;
    int64_t raw[kRegs];
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
        const int i = u * BT + tid;
        raw[u] = topk_idx[i < base ? i : last];
    }
    int c0, c1, b0, b1;
    ll_slice<kFP8>(V, ny, yb, c0, c1, b0, b1);
    const u32x4 first = ll_first<kFP8, kRows>(x, t, V, c0, c1, b0, b1);
    // Only now are the ids looked at: without these empty (volatile) uses the
    // compiler tests each id right after its load, which makes every later
    // load -- the row slice's too -- wait for it.
    asm volatile("" : "+v"(own_raw));
    int ids[kRegs];
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
        asm volatile("" : "+v"(raw[u]));
        ids[u] = u * BT + tid < base ? ll_valid_id(raw[u], E) : -1;
    }
    const int own = lane < K ? ll_valid_id(own_raw, E) : -1;
    bool live = own >= 0;
    if (rank_mask != nullptr && live)
        live = rank_mask[ll_rank(own, epr)] == 0;
    const int cell0 = live ? ll_cell(own, epr, R, S, 0) : -1;

    // lane k: matches of pair k's expert among this wave's entries (mine),
    // and among the token's pairs before k (dup)
    // Eight pairs per round, with no branch among them, so that their
    // readlane -> compare -> count chains overlap.  Rounds may run past K
    // (never past lane 63: K <= 64 and rounds start at multiples of 8); those
    // counts land in lanes >= K, which never read them.
    int mine = 0, dup = 0;
    for (int k0 = 0; k0 < K; k0 += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + j;
            const int ek = ll_readlane(own, k);
            int c = 0;
#pragma unroll
            for (int u = 0; u < kRegs; ++u)
                c += ll_count(ids[u] == ek);
            const int d = __popcll(__builtin_amdgcn_ballot_w64(own == ek) & ((1ull << k) - 1));
            mine = lane == k ? c : mine;
            dup = lane == k ? d : dup;
        }
    }
    if (lane < K)
        s_part[lane][wid] = mine;
    __syncthreads();

    int cell = -1, slot = -1;
    if (lane < K && live) {
        int cnt = dup;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            cnt += s_part[lane][w];
        if (cnt < S) {
            slot = cnt;
            cell = cell0 + cnt;
        }
    }
    if (yb == 0 && wid == 0 && lane < K) {
        topk_slot[base + lane] = slot;
        if (cell >= 0)
            src_info[cell] = t;
    }
    if (!kRows)
        return;
    ll_store_slice<kFP8, BT>(x, t, V, K, cell, first, c0, c1, b0, b1, packed_x, packed_q,
                             packed_scale);
}

// The one-launch kernel for a table of TK entries: kRegs = TK / BT rounded
// up to a power of two.
template <bool kFP8, int BT, bool kRows>
auto ll_tok_kernel_for(int64_t TK)
{
    const int64_t regs = (TK + BT - 1) / BT;
    return regs <= 1   ? ll_dispatch_tok_kernel<kFP8, BT, kRows, 1>
           : regs <= 2 ? ll_dispatch_tok_kernel<kFP8, BT, kRows, 2>
           : regs <= 4 ? ll_dispatch_tok_kernel<kFP8, BT, kRows, 4>
                       : ll_dispatch_tok_kernel<kFP8, BT, kRows, kLLTokPairs / BT>;
}

// Packed rows are read once by the combine.
__device__ __forceinline__ u32x4 ll_load_row(const u32x4 *p) { return *p; }

// The pairs' cells and weights for the combines: lane k < K of every wave
// holds pair (t, k)'s cell (-1: masked, dropped, or on a rank masked now)
// and its weight.
__device__ __forceinline__ void ll_pair_cells(int64_t t, int K, int E, int R, int epr, int S,
                                              const int64_t *__restrict__ topk_idx,
                                              const float *__restrict__ topk_weights,
                                              const int32_t *__restrict__ topk_slot,
                                              const int32_t *__restrict__ rank_mask, int &cell,
                                              float &w)
{
    const int lane = threadIdx.x & (kWave - 1);
    cell = -1;
    w = 0.0f;
    if (lane < K) {
        const int e = ll_valid_id(topk_idx[t * K + lane], E);
        const int s = topk_slot[t * K + lane];
        w = topk_weights[t * K + lane];
        bool ok = e >= 0 && s >= 0 && s < S;
        if (ok && rank_mask != nullptr)
            ok = rank_mask[e / epr] == 0;
        cell = ok ? ll_cell(e, epr, R, S, s) : -1;
    }
}

// One workgroup per (token, row slice), the dispatch's slices in the
// dispatch's order (kTokBlock).  Each wave resolves the token's K cells
// itself (lanes 0..K-1, no LDS, no barrier); each lane then issues its K
// loads before the fused multiply-adds, which run in ascending slot order
// from +0.
__global__ __launch_bounds__(kTokBlock) void ll_combine_kernel(
    const u32x4 *__restrict__ packed_y, int V, int K, int E, int R, int epr, int S, int ny,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    const int32_t *__restrict__ topk_slot, const int32_t *__restrict__ rank_mask,
    u32x4 *__restrict__ out)
{
    const int64_t t = blockIdx.x / ny;
    int c0, c1, b0, b1;
    ll_slice<false>(V, ny, int(blockIdx.x - t * ny), c0, c1, b0, b1);
    const int idx = c0 + threadIdx.x;  // this lane's vector of the row
    int cell;
    float w;
    ll_pair_cells(t, K, E, R, epr, S, topk_idx, topk_weights, topk_slot, rank_mask, cell, w);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = 0.0f;

    constexpr int kGroup = 8;
    for (int k0 = 0; k0 < K; k0 += kGroup) {
        u32x4 v[kGroup];
        int ck[kGroup];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            ck[g] = k0 + g < K ? ll_readlane(cell, k0 + g) : -1;
            v[g] = (ck[g] >= 0 && idx < c1) ? ll_load_row(packed_y + int64_t(ck[g]) * V + idx)
                                            : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            if (ck[g] >= 0) {
                const float wk = __int_as_float(ll_readlane(__float_as_int(w), k0 + g));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = __builtin_fmaf(wk, bf16_lo(v[g][q]), acc[2 * q]);
                    acc[2 * q + 1] = __builtin_fmaf(wk, bf16_hi(v[g][q]), acc[2 * q + 1]);
                }
            }
        }
    }
    if (idx < c1) {
        u32x4 rv;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            rv[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        out[t * V + idx] = rv;
    }
}

// The combine of an FP8 payload (codes and per-128-element-block scales, as
// the FP8 dispatch stores them).  A lane takes 8 elements of the row (one
// 8-byte word of codes per cell); each code is decoded exactly with the
// packed hardware conversion (checked against the e4m3 definition for all
// 256 codes), multiplied by its block's scale in fp32, and added with the
// same fma sum in ascending k as the bf16 combine.  Workgroups as in the
// bf16 combine: (token, slice of blocks), the FP8 dispatch's slices in its
// order; lane j of a slice takes group 16 * b0 + j, as in the dispatch.
__global__ __launch_bounds__(kTokBlock) void ll_combine_fp8_kernel(
    const uint2 *__restrict__ packed_q, const float *__restrict__ packed_scale, int V, int K,
    int E, int R, int epr, int S, int ny, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ topk_slot,
    const int32_t *__restrict__ rank_mask, u32x4 *__restrict__ out)
{
    const int64_t t = blockIdx.x / ny;
    int c0, c1, b0, b1;
    ll_slice<true>(V, ny, int(blockIdx.x - t * ny), c0, c1, b0, b1);
    const int idx = 16 * b0 + threadIdx.x;  // 8-element group of the row
    const int lim = 16 * b1;
    const int nb = V / 16;  // 128-element blocks per row
    int cell;
    float w;
    ll_pair_cells(t, K, E, R, epr, S, topk_idx, topk_weights, topk_slot, rank_mask, cell, w);
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = 0.0f;

    constexpr int kGroup = 8;
    for (int k0 = 0; k0 < K; k0 += kGroup) {
        uint2 c[kGroup];
        float sc[kGroup];
        int ck[kGroup];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            ck[g] = k0 + g < K ? ll_readlane(cell, k0 + g) : -1;
            const bool live = ck[g] >= 0 && idx < lim;
            c[g] = live ? packed_q[int64_t(ck[g]) * V + idx] : make_uint2(0, 0);
            sc[g] = live ? packed_scale[int64_t(ck[g]) * nb + idx / 16] : 0.0f;
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            if (ck[g] >= 0) {
                const float wk = __int_as_float(ll_readlane(__float_as_int(w), k0 + g));
                const uint32_t words[2] = {c[g].x, c[g].y};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(words[h]), false);
                    const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(words[h]), true);
                    acc[4 * h + 0] = __builtin_fmaf(wk, d01[0] * sc[g], acc[4 * h + 0]);
                    acc[4 * h + 1] = __builtin_fmaf(wk, d01[1] * sc[g], acc[4 * h + 1]);
                    acc[4 * h + 2] = __builtin_fmaf(wk, d23[0] * sc[g], acc[4 * h + 2]);
                    acc[4 * h + 3] = __builtin_fmaf(wk, d23[1] * sc[g], acc[4 * h + 3]);
                }
            }
        }
    }
    if (idx < lim) {
        u32x4 rv;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            rv[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        out[t * V + idx] = rv;
    }
}

std::atomic<int> g_ll_mode{0};  // 0 automatic, 1 slot scan + copy, 2 one launch when it fits

}  // namespace

bool set_ll_tuning(int mode)
{
    if (mode < 0 || mode > 2)
        return false;
    g_ll_mode = mode;
    return true;
}

// Row slices per token for workgroups of bt threads: about bt vectors
// (bf16) or bt / 16 blocks (fp8) each, one per lane or 16-lane group.
int ll_slices(int V, bool fp8, bool rows, int bt)
{
    if (!rows)
        return 1;
    return fp8 ? (V / 16 + bt / 16 - 1) / (bt / 16) : (V + bt - 1) / bt;
}

hipError_t launch_ll_dispatch(const ep_dims &d, int num_slots, const void *x,
                              const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                              void *packed_q, float *packed_scale, int32_t *packed_count,
                              int32_t *src_info, int32_t *topk_slot, hipStream_t stream)
{
    const int T = d.num_tokens, K = d.num_topk, E = d.num_experts, R = d.num_ranks;
    const int V = d.hidden / 8;
    const bool fp8 = packed_q != nullptr;
    const bool rows = fp8 || packed_x != nullptr;
    const int64_t TK = int64_t(T) * K;
    if (g_ll_mode.load() != 1 && TK <= kLLTokPairs) {
        constexpr int BT = kTokBlock;
        const int ny = ll_slices(V, fp8, rows, BT);
        const int64_t blocks = int64_t(T) * ny + (E + BT / kWave - 1) / (BT / kWave);
        if (log_enabled())
            log_launch("ll_dispatch one-launch T=%d H=%d K=%d E=%d: slices=%d blocks=%lld%s", T,
                       d.hidden, K, E, ny, (long long)blocks, fp8 ? " fp8" : "");
        auto tk = fp8    ? ll_tok_kernel_for<true, BT, true>(TK)
                  : rows ? ll_tok_kernel_for<false, BT, true>(TK)
                         : ll_tok_kernel_for<false, BT, false>(TK);
        hipLaunchKernelGGL(tk, dim3(unsigned(blocks)), dim3(BT), 0, stream,
                           static_cast<const u32x4 *>(x), T, V, K, E, R, E / R, num_slots, ny,
                           topk_idx, rank_mask, static_cast<u32x4 *>(packed_x),
                           static_cast<uint2 *>(packed_q), packed_scale, packed_count, src_info,
                           topk_slot);
        return hipGetLastError();
    }
    const int ny = ll_slices(V, fp8, rows, kTokBlock);
    if (log_enabled())
        log_launch("ll_dispatch slot scan + copy T=%d H=%d K=%d E=%d: slot blocks=%d copy "
                   "blocks=%lld%s",
                   T, d.hidden, K, E, E, rows ? (long long)T * ny : 0LL, fp8 ? " fp8" : "");
    const int64_t per_thread = (TK + kSlotBlock - 1) / kSlotBlock;
    auto sk = per_thread <= 2   ? ll_slot_kernel<2>
              : per_thread <= 4 ? ll_slot_kernel<4>
              : per_thread <= 8 ? ll_slot_kernel<8>
                                : ll_slot_kernel<kSlotMaxHold>;
    hipLaunchKernelGGL(sk, dim3(E), dim3(kSlotBlock), 0, stream, T, K, E, R, E / R, num_slots,
                       topk_idx, rank_mask, packed_count, src_info, topk_slot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !rows || T == 0)
        return e;
    auto ck = fp8 ? ll_copy_kernel<true> : ll_copy_kernel<false>;
    hipLaunchKernelGGL(ck, dim3(unsigned(int64_t(T) * ny)), dim3(kTokBlock), 0, stream,
                       static_cast<const u32x4 *>(x), V, K, E, R, E / R, num_slots, ny, topk_idx,
                       topk_slot, static_cast<u32x4 *>(packed_x), static_cast<uint2 *>(packed_q),
                       packed_scale);
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
    const int ny = ll_slices(V, true, true, kTokBlock);
    if (log_enabled())
        log_launch("ll_combine fp8 T=%d H=%d K=%d: slices=%d blocks=%lld", d.num_tokens,
                   d.hidden, d.num_topk, ny, (long long)d.num_tokens * ny);
    hipLaunchKernelGGL(ll_combine_fp8_kernel, dim3(unsigned(int64_t(d.num_tokens) * ny)),
                       dim3(kTokBlock), 0, stream, static_cast<const uint2 *>(packed_q),
                       packed_scale, V, d.num_topk, E, R, E / R, num_slots, ny, topk_idx,
                       topk_weights, topk_slot, rank_mask, static_cast<u32x4 *>(out));
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
    const int ny = ll_slices(V, false, true, kTokBlock);
    if (log_enabled())
        log_launch("ll_combine T=%d H=%d K=%d: slices=%d blocks=%lld", d.num_tokens, d.hidden,
                   d.num_topk, ny, (long long)d.num_tokens * ny);
    hipLaunchKernelGGL(ll_combine_kernel, dim3(unsigned(int64_t(d.num_tokens) * ny)),
                       dim3(kTokBlock), 0, stream, static_cast<const u32x4 *>(packed_y), V,
                       d.num_topk, E, R, E / R, num_slots, ny, topk_idx, topk_weights, topk_slot,
                       rank_mask, static_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace ep

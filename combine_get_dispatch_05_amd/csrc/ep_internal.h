// ep_internal.h -- declarations shared by the gfx950 kernels and the host
// runtime of libep.so.  Not part of the public ABI (that is include/ep.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// 16-byte vector: the unit of every token-row load and store (rows are whole
// int4 vectors, as the runtime's alignment rule requires).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxRanks = 512;     // NW <= 8 64-bit rank-mask words
constexpr int kMaxTopk = 64;
constexpr int kMaxExperts = 8192;  // per-block expert histogram lives in LDS
constexpr int kMaxChannels = 4096;
constexpr int kMaxLLSlots = 4096;  // slots per low-latency expert cell list
constexpr int64_t kMaxTokens = int64_t(1) << 24;
constexpr int kMaxHidden = 1 << 20;

// Device pointers of one layout (all inside a handle's arena).  The first
// kLayoutCtrBytes of every arena hold the one-launch layout's counters,
// zeroed when the arena is allocated and only ever increased after that.
constexpr int kArenaFields = 17;
constexpr size_t kLayoutCtrBytes = 256;
struct LayoutBufs {
    uint64_t *layout_ctr;                // [4] tickets, count units done, count blocks done, wait-timeout flag
    int32_t *num_tokens_per_rank;        // [R]
    int32_t *num_tokens_per_expert;      // [E]
    uint8_t *is_token_in_rank;           // [T][R]
    int32_t *rank_prefix_matrix;         // [R]
    int32_t *channel_prefix_matrix;      // [R][C]
    int32_t *recv_channel_prefix_matrix; // [R][C]
    int32_t *send_head;                  // [T][R]
    int32_t *recv_src_idx;               // [T*Kmax]
    int32_t *dst_row;                    // [T][Kmax] packed rows of t, ascending rank, -1 padded
    int32_t *dst_rank;                   // [T][Kmax] their ranks
    uint64_t *wave_mask;                 // [nW][R] ballot of "token hits r" per 64-token wave
    int32_t *wave_base;                  // [nW][R] hits of r in earlier waves of the same block
    int32_t *blk_count;                  // [nB][R] block totals (exclusive bases after a scan kernel)
    int32_t *blk_ecount;                 // [nB][E] per-block expert counts
    int64_t *num_recv;                   // [1] N
    uint64_t *topk_hash;                 // [2] hash of the layout's topk_idx, and of a later one
};

struct LayoutShape {
    int T, K, E, R, C, epr, kmax, nW, nB;
    bool fused;  // one-launch layout (count blocks of 256 tokens), else two kernels (512)
};

// allow_fused: the one-launch layout may be chosen (it needs the arena's
// counter bookkeeping, so only handle arenas allow it).
LayoutShape layout_shape(const ep_dims &d, bool allow_fused = true);
// Byte offsets of every LayoutBufs field inside one arena; returns the total.
size_t layout_arena_bytes(const LayoutShape &s, size_t off[kArenaFields]);
LayoutBufs layout_bufs_at(void *base, const size_t off[kArenaFields]);

// EP_LOG=1 in the environment: one line per kernel launch on stderr with its
// launch geometry (read at every call).
bool log_enabled();
void log_launch(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

// How far an arena's one-launch layout counters have advanced: the tickets
// and done marks of every layout launched in it so far (host-side, kept with
// the arena; stream order makes each launch start where the last one ended).
struct LayoutCounters {
    uint64_t tickets = 0;
    uint64_t done = 0;
    uint64_t counted = 0;  // count blocks that summed into the early N
};

// rank_mask [R] int32 (nullable): nonzero ranks are masked.  num_recv_host
// (nullable): pinned, coherent host memory that also receives N, exactly
// once, so that a caller waiting for N can poll it instead of copying it
// back.  On the two-kernel path the count kernel's last block stores it, as
// soon as the counts are known and before the positions are.
hipError_t launch_layout(const LayoutShape &s, const int64_t *topk_idx, const int32_t *rank_mask,
                         const LayoutBufs &b, int64_t *num_recv_host, LayoutCounters &lc,
                         hipStream_t stream);

hipError_t launch_dispatch(const LayoutShape &s, int hidden, const void *x, const LayoutBufs &b,
                           const int64_t *topk_idx, const float *topk_weights, void *recv_x,
                           int64_t *recv_topk_idx, float *recv_topk_weights, hipStream_t stream);

hipError_t launch_combine(const LayoutShape &s, int hidden, const void *y, const LayoutBufs &b,
                          const float *recv_topk_weights, const void *bias0, const void *bias1,
                          const int32_t *rank_mask, void *out, float *combined_topk_weights,
                          hipStream_t stream);

// packed_q (nullable) selects the FP8 variant: codes [cells][H] bytes and
// packed_scale [cells][H/128]; packed_x is then unused.
hipError_t launch_ll_dispatch(const ep_dims &d, int num_slots, const void *x,
                              const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                              void *packed_q, float *packed_scale, int32_t *packed_count,
                              int32_t *src_info, int32_t *topk_slot, hipStream_t stream);

hipError_t launch_ll_combine(const ep_dims &d, int num_slots, const void *packed_y,
                             const int64_t *topk_idx, const float *topk_weights,
                             const int32_t *topk_slot, const int32_t *rank_mask, void *out,
                             hipStream_t stream);
// packed_q: e4m3 codes [cells][H] bytes, packed_scale [cells][H/128].
hipError_t launch_ll_combine_fp8(const ep_dims &d, int num_slots, const void *packed_q,
                                 const float *packed_scale, const int64_t *topk_idx,
                                 const float *topk_weights, const int32_t *topk_slot,
                                 const int32_t *rank_mask, void *out, hipStream_t stream);

// Order-independent 64-bit hash of n top-k ids into *out (debug check).
hipError_t launch_topk_hash(const int64_t *topk_idx, int64_t n, uint64_t *out, hipStream_t stream);

hipError_t launch_mask_set(int32_t *mask, int num_ranks, int rank, int value, hipStream_t stream);

hipError_t launch_lb_reduce_grads(const void *redundant_grads, void *expert_grads,
                                  const int64_t *mapping, int num_replicas, int num_experts,
                                  int64_t elems, hipStream_t stream);

hipError_t launch_lb_prefetch_weights(const void *expert_weights, void *redundant_weights,
                                      const int64_t *mapping, int num_replicas, int num_experts,
                                      int64_t elems, hipStream_t stream);

// Launch-shape overrides (never change results).  (-1, ...) restores the
// default choice.  Return false for a shape that is not compiled in.
bool set_dispatch_tuning(int g, int vpt, int code);
bool set_combine_tuning(int g, int vpt, int u);
// Low-latency dispatch variant: 0 automatic (one launch for T*K <= 4096,
// else slot scan + token-major copy), 1 slot scan + copy always, 2 one
// launch whenever T*K allows.
bool set_ll_tuning(int mode);
// Layout: 0 automatic (the count and position kernels), 1 those kernels
// always, 2 one launch whenever it fits (up to 8192 tokens).  Read when a
// handle is made.
bool set_layout_tuning(int mode);
int dispatch_tuning_count();
void dispatch_tuning_at(int i, int *g, int *vpt, int *code);
int combine_tuning_count();
void combine_tuning_at(int i, int *g, int *vpt, int *u);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 round to nearest, ties to even: add just under half of the
// dropped 16-bit fraction, plus one when the kept lsb is odd, then truncate.
// A mantissa carry correctly bumps the exponent.  NaN is kept quiet.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt()
{
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace ep

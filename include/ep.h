/*
 * ep.h -- C ABI of the MI355X (gfx950) expert-parallel layout / dispatch /
 * combine library (libep.so).
 *
 * The operations follow these pages:
 *   [P1] "DeepEP Buffer Class API for Expert Parallel Communication:
 *        Architecture and Usage": "Configuration and Layout Helpers"
 *        (get_dispatch_layout), "Dispatch Operation", "Combine Operation",
 *        "IB-GDA Kernels" (low_latency_dispatch / low_latency_combine),
 *        "Explicit Resource Cleanup" (destroy) and the FAQ on the handle.
 *   [P3] DeepEP-Lib "Core Implementation" (C++ runtime): "Memory Alignment
 *        and Validation" (int4-multiple rows, buffer alignment).
 *   [P4] "How DeepEP Optimizes Handle Reuse for Repeated Dispatches": "What
 *        the Handle Contains", "Fast Path Dispatch with Handle Reuse",
 *        "Performance Contract and Constraints".
 *   [P5] "Chapter 10, V2: buffers beyond EP", section 10.2 (load-balance
 *        operations over redundant experts).
 *
 * The R destination ranks are logical partitions of this GPU's memory: a
 * "segment" is a contiguous range of rows of one caller buffer.  Nothing here
 * talks to another GPU.
 *
 * Conventions for every entry point
 *   - Memory: every array argument is a DEVICE pointer owned by the caller,
 *     except the ones documented as host pointers.  The library never frees
 *     caller memory.  The handle is the only library-owned memory.
 *   - Streams: `stream` is a hipStream_t (NULL = the legacy default stream).
 *     All device work is enqueued on it, in order; no call synchronizes the
 *     host unless its documentation says so.
 *   - Layouts are dense row-major.  bf16 tensors are 16-bit words.  topk_idx
 *     is int64 with -1 for a masked slot; weights are fp32.
 *   - Expert e belongs to rank e / (E/R) as local expert e % (E/R).
 *   - Alignment ([P3]): token-row pointers (x, recv_x, y, out, bias0, bias1,
 *     packed_x, packed_y, load-balance tensors) must be 16-byte aligned, and
 *     hidden*2 must be a multiple of 16 (rows are whole int4 vectors); int64
 *     arrays 8-byte, others 4-byte aligned.  Violations return EP_ERR_ALIGN
 *     before any work is enqueued.
 *   - Expert ids outside [-1, E) are invalid input.  The kernels ignore such
 *     slots (treat them as masked) so that no access leaves its buffer.
 *   - Errors: every int-returning call returns an ep_status.  On any error no
 *     work has been enqueued and no output pointer argument was written,
 *     except as noted.  Host-side errors never throw across the ABI.
 *   - Environment (read by the library, never required):
 *       EP_LOG=1     one line per kernel launch on stderr with its launch geometry;
 *       EP_TRACE=1   a roctx range around every entry point (rocprofv3 marker trace);
 *       EP_CHECK=1   the handle-reuse table check of ep_dispatch;
 *       EP_TUNE_DISPATCH / EP_TUNE_COMBINE   initial launch-shape overrides (ep_set_tuning).
 *   - Concurrency: calls may run on different streams concurrently as long
 *     as they do not write the same caller memory.  One handle may be read by
 *     several calls at once; it must not be freed while they are in flight
 *     on other streams than its last one (the freed memory is reused only by
 *     work on the handle's last stream).
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ep_stream_t; /* a hipStream_t */

typedef enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID = 1,  /* bad dimension, NULL where required, forbidden argument mix */
    EP_ERR_ALIGN = 2,    /* pointer or row-size alignment rule broken */
    EP_ERR_CAPACITY = 3, /* caller buffer has fewer rows than the result needs */
    EP_ERR_HANDLE = 4,   /* handle does not match the dims, or NULL handle */
    EP_ERR_HIP = 5,      /* a HIP runtime call failed (see ep_last_hip_error) */
    EP_ERR_NOMEM = 6,    /* device or host allocation failed */
    EP_ERR_TOO_LARGE = 7 /* needs more than ep_get_dispatch_layout_noalloc's static scratch */
} ep_status;

/* Problem sizes.  Limits: 0 <= num_tokens <= 2^24; hidden > 0, hidden % 8 == 0,
 * hidden <= 2^20; 1 <= num_topk <= 64; 1 <= num_ranks <= 512;
 * num_experts % num_ranks == 0, num_experts <= 8192; num_channels >= 1,
 * num_channels <= 4096. */
typedef struct ep_dims {
    int32_t num_tokens;   /* T */
    int32_t hidden;       /* H, bf16 elements per token row */
    int32_t num_topk;     /* K */
    int32_t num_experts;  /* E */
    int32_t num_ranks;    /* R */
    int32_t num_channels; /* C: channels are ceil(T/C)-token contiguous ranges */
} ep_dims;

/* Opaque, library-owned dispatch layout ("handle" of [P4] "What the Handle
 * Contains"): rank_prefix_matrix, channel_prefix_matrix,
 * recv_channel_prefix_matrix, recv_src_idx, is_token_in_rank, send_head, the
 * per-rank and per-expert counts, the dims, and per-token destination-row
 * lists.  Immutable once created; freed by ep_handle_free. */
typedef struct ep_handle ep_handle;

/* Caller-owned device outputs of the layout.  Any field may be NULL (not
 * wanted).  Shapes:
 *   num_tokens_per_rank        int32 [R]    tokens that go to rank r
 *   num_tokens_per_expert      int32 [E]    (token, slot) pairs naming e
 *   is_token_in_rank           uint8 [T][R] 1 iff t goes to r
 *   rank_prefix_matrix         int32 [R]    inclusive prefix of num_tokens_per_rank;
 *                                           segment r starts at row [r-1] (0 for r = 0),
 *                                           N = [R-1] rows in total
 *   channel_prefix_matrix      int32 [R][C] tokens of rank r before the end of channel c
 *   recv_channel_prefix_matrix int32 [R][C] tokens of rank r before the start of channel c
 *   send_head                  int32 [T][R] row of t inside segment r, -1 if none
 *   recv_src_idx               int32 [recv_src_cap] source token of packed row i, i < N
 */
typedef struct ep_layout_out {
    int32_t *num_tokens_per_rank;
    int32_t *num_tokens_per_expert;
    uint8_t *is_token_in_rank;
    int32_t *rank_prefix_matrix;
    int32_t *channel_prefix_matrix;
    int32_t *recv_channel_prefix_matrix;
    int32_t *send_head;
    int32_t *recv_src_idx;
    int64_t recv_src_cap; /* rows available in recv_src_idx */
} ep_layout_out;

/* Largest possible row count N of a dispatch: T * min(K, R). */
int64_t ep_max_recv_rows(const ep_dims *dims);

/*
 * [P1] "Configuration and Layout Helpers": compute the token-to-rank layout
 * of topk_idx [T][K] on the GPU, before any token data moves.
 *
 * out (nullable): fields that are non-NULL receive copies of the layout.  If
 *   out->recv_src_idx is non-NULL and recv_src_cap < ep_max_recv_rows(), the
 *   call waits for N (the layout's count kernel stores it into pinned host
 *   memory, which the host polls; the positions may still be being written
 *   when it returns) and returns EP_ERR_CAPACITY if N > recv_src_cap;
 *   then no output in `out` is written and no handle is returned (*handle_out
 *   is left unchanged; the layout's memory returns to the pool).
 * handle_out (nullable): receives a new handle holding the layout.  Such a
 *   handle may be given to one ep_dispatch together with the same topk_idx
 *   (the "pre-computed layout" of [P1] "Dispatch Operation").
 * rank_mask [R] int32 (nullable; [P1] "Dynamic Rank Masking", nonzero =
 *   masked): every slot whose expert lives on a masked rank is treated as a
 *   masked slot, so a masked rank gets no tokens and its experts count 0.
 *   The mask is read on the device when the layout kernels run.
 * No host synchronization unless noted above.
 */
int ep_get_dispatch_layout(const ep_dims *dims, const int64_t *topk_idx, const int32_t *rank_mask,
                           ep_layout_out *out, ep_handle **handle_out, ep_stream_t stream);

/*
 * ep_get_dispatch_layout for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same layout, written into `out`, with no handle, no hipMalloc / hipFree /
 * host allocation and no host synchronization.  The layout kernels write the
 * caller's buffers directly; their scratch (and any output field left NULL)
 * lives in one static device array of EP_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and give
 * undefined results; calls in one stream's order are fine.  Nothing in the
 * array needs to start at zero.
 *   out: required.  Fields as for ep_get_dispatch_layout; recv_src_idx, when
 *     non-NULL, needs recv_src_cap >= ep_max_recv_rows() (EP_ERR_CAPACITY
 *     otherwise: N is not read back).  send_head must be 16-byte aligned and
 *     is_token_in_rank 4-byte aligned (EP_ERR_ALIGN), since the kernels store
 *     them 4 ranks at a time.
 *   The layout always takes the count and position kernels (the one-launch
 *   layout of the "layout" tuning knob is not used here).
 * A problem whose scratch would exceed EP_NOALLOC_SCRATCH_BYTES returns
 * EP_ERR_TOO_LARGE before anything is enqueued.
 */
#define EP_NOALLOC_SCRATCH_BYTES (32u << 20)
int ep_get_dispatch_layout_noalloc(const ep_dims *dims, const int64_t *topk_idx,
                                   const int32_t *rank_mask, ep_layout_out *out,
                                   ep_stream_t stream);

/*
 * [P1] "Dispatch Operation" and [P4] "Fast Path Dispatch with Handle Reuse":
 * pack token rows x [T][H] (bf16) into R contiguous per-rank segments of
 * recv_x [recv_cap][H] in token order: row S[r] + send_head[t][r] receives
 * x[t] for every rank r that t goes to.
 *
 *   *handle == NULL       fresh dispatch: topk_idx is required; the layout is
 *                         computed and a new handle is stored in *handle.
 *   handle from ep_get_dispatch_layout and not yet used by a dispatch:
 *                         the layout is reused; topk_idx / topk_weights may
 *                         be given and must be the table the layout came from.
 *   handle returned by an earlier dispatch (cached fast path):
 *                         topk_idx and topk_weights must be NULL
 *                         (EP_ERR_INVALID otherwise); only rows are packed.
 *
 * recv_topk_idx [recv_cap][K] int64 (nullable, needs topk_idx): slot k of
 *   packed row (t, r) holds e - r*(E/R) when slot k of t is valid and its
 *   expert e lives on r, else -1.
 * recv_topk_weights [recv_cap][K] fp32 (nullable, needs topk_weights): the
 *   slot's weight in the same case, else 0.
 * recv_x (nullable): NULL skips the row copy (layout / size query only).
 * recv_cap: rows available in recv_x / recv_topk_*.  If it is below N the
 *   call returns EP_ERR_CAPACITY.  When recv_cap >= ep_max_recv_rows() no
 *   host synchronization is needed to check it.
 * num_recv (HOST pointer, nullable): receives N; asking for it waits once
 *   per handle (later calls use the cached value).  On a fresh dispatch the
 *   layout's count kernel stores N into pinned host memory, which the host
 *   polls (no copy is enqueued, and the call does not wait for the position
 *   kernel); on a handle made earlier N is copied there once and polled.
 * On any error of a fresh dispatch the new handle is released again and
 *   *handle is left NULL (the layout may already be enqueued; its memory
 *   returns to the pool in stream order).
 * Debug check ([P4] "Performance Contract and Constraints": a layout is only
 *   valid for the table it came from): with EP_CHECK=1 in the environment,
 *   ep_get_dispatch_layout stores a 64-bit hash of topk_idx in the handle,
 *   and a dispatch given that handle together with a topk_idx hashes it and
 *   reads both hashes back (one stream synchronization); a different table
 *   returns EP_ERR_INVALID before anything is packed.
 * rank_mask [R] int32 (nullable): as for ep_get_dispatch_layout; used only
 *   by a fresh dispatch (the layout it computes).  A handle already holds
 *   its layout, so a non-NULL rank_mask with *handle != NULL returns
 *   EP_ERR_INVALID.
 * dims must equal the handle's dims except hidden, which may differ.
 */
int ep_dispatch(const ep_dims *dims, const void *x, const int64_t *topk_idx,
                const float *topk_weights, const int32_t *rank_mask, ep_handle **handle,
                void *recv_x, int64_t *recv_topk_idx, float *recv_topk_weights,
                int64_t recv_cap, int64_t *num_recv, ep_stream_t stream);

/*
 * [P1] "Combine Operation": addition-based reduction of the packed rows
 * y [y_rows][hidden] (bf16, same segment layout as the dispatch that made
 * handle) back to token order:
 *   out[t] = bf16_rne( sum over ranks r ascending that t went to of
 *                      fp32(y[S[r] + send_head[t][r]])
 *                      + fp32(bias0[t]) + fp32(bias1[t]) ),
 *   fp32 accumulation starting at +0, in that order; a token that went
 *   nowhere gets the bias sum (+0 without bias).
 * bias0, bias1 [T][hidden] bf16 (each nullable): the optional bias terms of
 *   the same section, added after the rank sum, before the one rounding.
 * recv_topk_weights [y_rows][K] fp32 (nullable) and combined_topk_weights
 * [T][K] fp32 (nullable, needs the former): the same ascending-rank fp32 sum
 * of the per-row weights (the reduced weights combine returns).
 * rank_mask [R] int32 (nullable; [P1] "Dynamic Rank Masking"): ranks masked
 *   now (nonzero) are left out of both sums, as if t had not gone there;
 *   the order of the remaining terms is unchanged.
 * y_rows below N returns EP_ERR_CAPACITY (checked without synchronizing
 * when y_rows >= ep_max_recv_rows(), else N is read once per handle).
 */
int ep_combine(ep_handle *handle, int32_t hidden, const void *y, int64_t y_rows,
               const float *recv_topk_weights, const void *bias0, const void *bias1,
               const int32_t *rank_mask, void *out, float *combined_topk_weights,
               ep_stream_t stream);

/*
 * [P1] "IB-GDA Kernels", low_latency_dispatch: stream every valid (token,
 * slot) pair straight into its expert's receive area.  With epr = E/R:
 *   packed_x  [epr][R][num_slots][H] bf16: cell (le, r, s) gets x[t] for the
 *             pair (t, k) naming expert r*epr + le whose slot is s
 *   packed_count [epr][R] int32: pairs routed to each expert
 *   src_info  [epr][R][num_slots] int32: source token of each used cell, -1
 *             for unused cells
 *   topk_slot [T][K] int32: slot s of pair (t, k), -1 when masked or dropped
 * Slots follow (token, slot) order.  Requires T <= num_slots
 * (EP_ERR_CAPACITY); pairs past num_slots (possible only when a token names
 * one expert twice) are dropped and still counted.  Unused packed_x cells
 * are not written.  packed_x may be NULL (metadata only).  No host sync.
 * rank_mask [R] int32 (nullable; [P1] "Dynamic Rank Masking"): nonzero
 *   marks a masked rank, whose experts receive nothing (count 0, no slots;
 *   their pairs get topk_slot -1), as if those slots were masked.
 */
int ep_ll_dispatch(const ep_dims *dims, int32_t num_slots, const void *x,
                   const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                   int32_t *packed_count, int32_t *src_info, int32_t *topk_slot,
                   ep_stream_t stream);

/*
 * ep_ll_dispatch with an FP8 payload ([P1] "IB-GDA Kernels": FP8 with
 * use_fp8, which the pages' code example sets on the dispatch).  Slots,
 * counts, src_info and topk_slot are exactly those of ep_ll_dispatch.
 * Every sent row is cut into 128-element blocks; per block
 *   amax = max(max |x|, 1e-4), q = e4m3(x * (448 / amax)), scale = amax / 448
 * in fp32, e4m3 being OCP FP8 E4M3 ("e4m3fn") with round to nearest even,
 * saturating at +-448.  x ~ q * scale.
 *   packed_q     [E/R][R][num_slots][H]     uint8 codes (8-byte aligned)
 *   packed_scale [E/R][R][num_slots][H/128] fp32
 * Requires hidden % 128 == 0 (EP_ERR_ALIGN).  Unused cells are not written.
 */
int ep_ll_dispatch_fp8(const ep_dims *dims, int32_t num_slots, const void *x,
                       const int64_t *topk_idx, const int32_t *rank_mask, void *packed_q,
                       float *packed_scale, int32_t *packed_count, int32_t *src_info,
                       int32_t *topk_slot, ep_stream_t stream);

/*
 * [P1] "IB-GDA Kernels", low_latency_combine: for every token,
 *   out[t] = bf16_rne(acc),  acc = fma(topk_weights[t][k], fp32(cell(t, k)), acc)
 * over k ascending, valid non-dropped slots only, from acc = +0, where cell
 * (t, k) is the packed_y row [le][r][topk_slot[t][k]] of the slot's expert.
 * packed_y has packed_x's layout; topk_slot comes from ep_ll_dispatch.
 * rank_mask [R] (nullable): pairs whose expert sits on a rank masked now
 * contribute nothing, whatever the dispatch did.  No host sync.
 */
int ep_ll_combine(const ep_dims *dims, int32_t num_slots, const void *packed_y,
                  const int64_t *topk_idx, const float *topk_weights,
                  const int32_t *topk_slot, const int32_t *rank_mask, void *out,
                  ep_stream_t stream);

/*
 * ep_ll_combine with an FP8 payload, the layout ep_ll_dispatch_fp8 writes
 * ([P1] "IB-GDA Kernels", FP8 with use_fp8; reading: the scales are applied
 * in the combine).  For every element of a cell:
 *   v = e4m3_decode(code) * scale[block]      (exact decode, one fp32 multiply)
 * then exactly the weighted sum of ep_ll_combine:
 *   out[t] = bf16_rne(acc),  acc = fma(topk_weights[t][k], v(cell(t, k)), acc)
 * over k ascending, valid non-dropped slots, from acc = +0.
 *   packed_q     [epr][R][num_slots][H] e4m3 codes (bytes), 8-byte aligned
 *   packed_scale [epr][R][num_slots][H/128] fp32
 * hidden must be a multiple of 128 (EP_ERR_ALIGN).  A NaN code gives NaN
 * terms.  rank_mask as for ep_ll_combine.  No host sync.
 */
int ep_ll_combine_fp8(const ep_dims *dims, int32_t num_slots, const void *packed_q,
                      const float *packed_scale, const int64_t *topk_idx,
                      const float *topk_weights, const int32_t *topk_slot,
                      const int32_t *rank_mask, void *out, ep_stream_t stream);

/* [P1] "Dynamic Rank Masking" on a caller-owned device mask rank_mask[R]
 * (0 active, 1 masked), stream-ordered like the other calls:
 *   ep_mask_update  set rank `rank` to masked (nonzero) or active (0)
 *   ep_mask_clean   set every rank active
 *   ep_mask_query   copy the mask to host_out[R] (HOST pointer); this call
 *                   synchronizes the stream. */
int ep_mask_update(int32_t *rank_mask, int32_t num_ranks, int32_t rank, int32_t masked,
                   ep_stream_t stream);
int ep_mask_clean(int32_t *rank_mask, int32_t num_ranks, ep_stream_t stream);
int ep_mask_query(const int32_t *rank_mask, int32_t num_ranks, int32_t *host_out,
                  ep_stream_t stream);

/*
 * Load balancing over redundant expert replicas ([P5] 10.2): replica j is a
 * copy of expert mapping[j] (mapping: int64 [num_replicas], device; entries
 * outside [0, num_experts) are ignored).  Tensors are bf16, one row of
 * elems_per_expert elements per expert / replica (elems % 8 == 0, 16-byte
 * aligned rows).
 *   ep_lb_prefetch_weights: redundant[j] = expert[mapping[j]] (bit copy).
 *   ep_lb_reduce_grads: for every expert e with replicas,
 *     expert[e] = bf16_rne(fp32(expert[e]) + sum over j ascending with
 *                          mapping[j] == e of fp32(redundant[j])),
 *     in place; experts without replicas are untouched.
 * num_replicas <= 65535.  No host sync.
 */
int ep_lb_prefetch_weights(const void *expert_weights, void *redundant_weights,
                           const int64_t *mapping, int32_t num_replicas, int32_t num_experts,
                           int64_t elems_per_expert, ep_stream_t stream);
int ep_lb_reduce_grads(const void *redundant_grads, void *expert_grads, const int64_t *mapping,
                       int32_t num_replicas, int32_t num_experts, int64_t elems_per_expert,
                       ep_stream_t stream);

/* Copy the handle's layout into caller buffers (fields may be NULL); same
 * shapes and capacity rule as ep_get_dispatch_layout. */
int ep_handle_copy_layout(ep_handle *handle, ep_layout_out *out, ep_stream_t stream);

/* N of the handle.  The first time, waits for the handle's last stream to
 * reach the copy of N into pinned host memory (work enqueued after it may
 * still be running when the call returns); later calls use the cached value. */
int ep_handle_num_recv(ep_handle *handle, int64_t *num_recv);

/* The handle's dims (host copy). */
int ep_handle_dims(const ep_handle *handle, ep_dims *dims);

/* Device bytes the handle holds (the print_memory_usage of the pages' V2.5
 * buffer base class). */
size_t ep_handle_nbytes(const ep_handle *handle);

/* [P1] "Explicit Resource Cleanup": release a handle.  NULL is a no-op.  The
 * memory returns to the library's per-device pool, tagged with the handle's
 * last stream; only a later handle made on that same stream reuses it, so
 * stream order puts every use of the memory before its reuse.  Nothing is
 * enqueued.
 * The pool is capped per device: at most EP_POOL_CAP_MB MiB (environment,
 * read once; default 256) and 64 arenas.  A free that takes the pool past
 * either limit synchronizes the device once (the only case in which this
 * call waits), returns the oldest arenas to HIP until the pool holds at most
 * half the byte cap and 32 arenas, and makes the arenas it keeps reusable by
 * handles on any stream (they are idle after that synchronization). */
void ep_handle_free(ep_handle *handle);

/* Release every pooled device allocation of the calling thread's current
 * device (synchronizes the device first).  Returns an ep_status. */
int ep_pool_trim(void);

/* The calling thread's current device's pool: bytes and arenas it keeps for
 * reuse, and its byte cap (each pointer nullable; HOST pointers).  Returns an
 * ep_status. */
int ep_pool_stats(size_t *kept_bytes, int32_t *kept_arenas, size_t *cap_bytes);

/* Launch-shape override for the pack ("dispatch") or the reduce ("combine")
 * kernels, process-wide, for every later call.  Results never depend on it.
 * a = lanes per group G, b = 16-byte vectors per lane VPT, c = a code for
 * the rest: dispatch X*10000 + S*1000 + NTL*100 + NTS*10 + P/256, combine
 * X*10000 + S*1000 + U*100 + NTL*10 + P/256, where X = 1 for the
 * destination-major (scatter) pack (the default) and the gather-form reduce
 * (G threads per workgroup, one vector each),
 * S = lane groups per token (row slices), NTS/NTL = nontemporal
 * stores/loads, U = rows in flight and P = persistent block count (0 = one
 * lane group per token slice).  ep_tuning_list enumerates the compiled-in
 * shapes.  a = b = c = -1 restores the default choice; a shape
 * that is not compiled in returns EP_ERR_INVALID.  The env vars
 * EP_TUNE_DISPATCH="G,VPT,c" and EP_TUNE_COMBINE="G,VPT,c" set the initial
 * override.
 * op "ll" picks the low-latency dispatch kernels (b = c = 0): a = 0 automatic
 * (one launch when T*K <= 4096, else a per-expert slot scan followed by a
 * token-major row copy), 1 slot scan + copy always, 2 one launch whenever
 * T*K <= 4096.  Both give identical results.
 * op "layout" picks the layout kernels (b = c = 0), for handles made
 * afterwards: a = 0 automatic (= 1), 1 the count and position kernels (a
 * scan kernel between them past 16384 tokens), 2 one launch whenever it fits
 * (up to 8192 tokens; measured slower than two launches on gfx950, kept for
 * callers that count launches).  Identical results. */
int ep_set_tuning(const char *op, int a, int b, int c);

/* Enumerate the compiled-in shapes of `op`: writes shape `index` (if in
 * range) to a, b, c and returns how many there are (-1 for an unknown op). */
int ep_tuning_list(const char *op, int index, int *a, int *b, int *c);

/* Static text of a status code. */
const char *ep_status_str(int status);

/* Text of the last HIP error seen by this thread (empty if none). */
const char *ep_last_hip_error(void);

/* ABI version: (major << 16) | minor.  2.0: rank_mask arguments of
 * ep_get_dispatch_layout, ep_dispatch and ep_combine; 2.1: ep_ll_combine_fp8;
 * 2.2: ep_pool_stats and the capped pool; 2.3: ep_get_dispatch_layout_noalloc
 * and EP_ERR_TOO_LARGE; 2.4: the destination-major dispatch and gather-form
 * combine tuning shapes (code X*10000). */
int ep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */

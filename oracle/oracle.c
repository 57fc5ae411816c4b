/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the expert-parallel
 * routing layout, dispatch pack and combine reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU baseline leg of
 * the benchmark use it.  It shares no code with the HIP library.
 *
 * Each function is the plain definition of the quantity it computes, written
 * from these pages:
 *   [P1] "DeepEP Buffer Class API for Expert Parallel Communication:
 *        Architecture and Usage", sections "Configuration and Layout Helpers",
 *        "Dispatch Operation", "Combine Operation", "IB-GDA Kernels" and the
 *        FAQ entry on the handle.
 *   [P3] DeepEP-Lib "Core Implementation" (C++ runtime), section "Memory
 *        Alignment and Validation".
 *   [P4] "How DeepEP Optimizes Handle Reuse for Repeated Dispatches",
 *        sections "What the Handle Contains" and "Fast Path Dispatch with
 *        Handle Reuse".
 * Where the pages leave a step open, the reading taken is stated next to the
 * code as "reading:".
 *
 * Conventions: topk_idx is int64 [T][K], -1 marks a masked slot.  Experts sit
 * in contiguous blocks of epr = E/R per rank (reading), so rank(e) = e / epr.
 * bf16 values are carried as uint16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 --- */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even from fp32 to bf16, from the IEEE-754 definition:
 * keep the top 16 bits; the 16 discarded bits are a fraction of one bf16 ulp;
 * add just under half an ulp, plus one more when the kept lsb is odd, so that
 * an exact tie rounds to the even neighbour.  A carry out of the mantissa
 * moves into the exponent, which is the correct rounding up to the next
 * binade (and to infinity past the largest finite value).  NaN keeps its sign
 * and payload top bits and gets the quiet bit set. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_f32_to_bf16(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(in[i]);
}

/* --------------------------------------------------------------- layout --- */

/* Channel c covers tokens [min(c*per, T), min((c+1)*per, T)) with
 * per = ceil(T / C).  Reading: "channels" are contiguous token ranges of equal
 * length, the last one short (or empty when C does not divide the tokens). */
static int64_t channel_end(int64_t c, int64_t T, int64_t C)
{
    int64_t per = (T + C - 1) / C;
    int64_t e = (c + 1) * per;
    return e < T ? e : T;
}

/*
 * The routing layout of [P1] "Configuration and Layout Helpers" plus the
 * handle matrices of [P4] "What the Handle Contains".
 *
 * Outputs (caller-allocated):
 *   num_tokens_per_expert[E]  number of (token, slot) pairs routed to e.
 *                             Reading: counted per slot, so an expert that a
 *                             token names twice counts twice.
 *   is_token_in_rank[T][R]    1 iff some valid slot of t names an expert of r.
 *   num_tokens_per_rank[R]    sum over t of is_token_in_rank[t][r].
 *   rank_prefix_matrix[R]     inclusive prefix of num_tokens_per_rank over
 *                             destination ranks; with one sender the matrix
 *                             has one row (reading).  Segment r of the packed
 *                             buffer starts at S[r] = rank_prefix_matrix[r-1].
 *   channel_prefix_matrix[R][C]       in-rank tokens before the end of
 *                             channel c (inclusive over channels, reading).
 *   recv_channel_prefix_matrix[R][C]  the exclusive version: in-rank tokens
 *                             before the start of channel c (reading).
 *   send_head[T][R]           position of t inside segment r in token order,
 *                             -1 when t does not go to r.
 *   recv_src_idx[N]           source token of each packed row: the inverse of
 *                             send_head, N = rank_prefix_matrix[R-1].
 * Returns N, or -1 on invalid arguments.
 */
int64_t oracle_layout(int64_t T, int64_t K, int64_t E, int64_t R, int64_t C,
                      const int64_t *topk_idx,
                      int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                      uint8_t *is_token_in_rank, int32_t *rank_prefix_matrix,
                      int32_t *channel_prefix_matrix, int32_t *recv_channel_prefix_matrix,
                      int32_t *send_head, int32_t *recv_src_idx, int64_t recv_src_cap)
{
    if (T < 0 || K < 1 || E < 1 || R < 1 || C < 1 || E % R != 0)
        return -1;
    int64_t epr = E / R;

    for (int64_t e = 0; e < E; ++e)
        num_tokens_per_expert[e] = 0;
    memset(is_token_in_rank, 0, (size_t)(T * R));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0)
                continue; /* masked slot: takes part in nothing */
            if (e >= E)
                return -1;
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + e / epr] = 1;
        }
    }

    for (int64_t r = 0; r < R; ++r) {
        int32_t n = 0;
        for (int64_t t = 0; t < T; ++t)
            n += is_token_in_rank[t * R + r];
        num_tokens_per_rank[r] = n;
    }

    int32_t acc = 0;
    for (int64_t r = 0; r < R; ++r) {
        acc += num_tokens_per_rank[r];
        rank_prefix_matrix[r] = acc;
    }
    int64_t N = acc;

    for (int64_t r = 0; r < R; ++r) {
        for (int64_t c = 0; c < C; ++c) {
            int64_t end = channel_end(c, T, C);
            int32_t n = 0;
            for (int64_t t = 0; t < end; ++t)
                n += is_token_in_rank[t * R + r];
            channel_prefix_matrix[r * C + c] = n;
        }
        for (int64_t c = 0; c < C; ++c)
            recv_channel_prefix_matrix[r * C + c] = c > 0 ? channel_prefix_matrix[r * C + c - 1] : 0;
    }

    for (int64_t r = 0; r < R; ++r) {
        int32_t pos = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (is_token_in_rank[t * R + r])
                send_head[t * R + r] = pos++;
            else
                send_head[t * R + r] = -1;
        }
    }

    if (recv_src_idx != NULL) {
        if (recv_src_cap < N)
            return -1;
        for (int64_t r = 0; r < R; ++r) {
            int64_t base = r > 0 ? rank_prefix_matrix[r - 1] : 0;
            for (int64_t t = 0; t < T; ++t)
                if (send_head[t * R + r] >= 0)
                    recv_src_idx[base + send_head[t * R + r]] = (int32_t)t;
        }
    }
    return N;
}

/* ------------------------------------------------------------- dispatch --- */

/*
 * Dispatch pack, [P1] "Dispatch Operation": every token row goes once to each
 * destination rank it hits, into that rank's contiguous segment, in token
 * order.  Row of (t, r) is S[r] + send_head[t][r].
 *
 * recv_topk_idx[row][k] is the slot's expert renumbered local to r
 * (e - r*epr) when the slot is valid and its expert lives on r, else -1;
 * recv_topk_weights[row][k] is the slot's weight in the same case, else 0
 * (reading of "topk_idx remapped to local experts and the matching weights").
 * Either topk output may be NULL.  x_new may differ from the x the layout was
 * built for: that is the handle-reuse dispatch of [P4] "Fast Path Dispatch
 * with Handle Reuse", which reuses send_head and rank_prefix_matrix.
 */
void oracle_dispatch(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R,
                     const uint16_t *x, const int64_t *topk_idx, const float *topk_weights,
                     const int32_t *rank_prefix_matrix, const int32_t *send_head,
                     uint16_t *recv_x, int64_t *recv_topk_idx, float *recv_topk_weights)
{
    int64_t epr = E / R;
    for (int64_t r = 0; r < R; ++r) {
        int64_t base = r > 0 ? rank_prefix_matrix[r - 1] : 0;
        for (int64_t t = 0; t < T; ++t) {
            int32_t p = send_head[t * R + r];
            if (p < 0)
                continue;
            int64_t row = base + p;
            if (recv_x != NULL)
                memcpy(recv_x + row * H, x + t * H, (size_t)H * sizeof(uint16_t));
            for (int64_t k = 0; k < K; ++k) {
                int64_t e = topk_idx != NULL ? topk_idx[t * K + k] : -1;
                int mine = e >= 0 && e / epr == r;
                if (recv_topk_idx != NULL)
                    recv_topk_idx[row * K + k] = mine ? e - r * epr : -1;
                if (recv_topk_weights != NULL)
                    recv_topk_weights[row * K + k] = mine ? topk_weights[t * K + k] : 0.0f;
            }
        }
    }
}

/* -------------------------------------------------------------- combine --- */

/*
 * Combine, [P1] "Combine Operation": an addition-based reduction of the rows
 * each token sent out, mapped back to the token with the handle.
 *   out[t][h] = bf16_rne( sum over r = 0..R-1 ascending, where t hit r, of
 *               f32(y[S[r] + send_head[t][r]][h]) )
 * The sum is sequential fp32 starting from +0 (reading: ascending rank order,
 * fp32 accumulation).  A token that hit no rank gets +0.
 * The optional weight output is the same reduction of recv_topk_weights,
 * kept in fp32 (the reduced weights the pages' combine returns).
 */
void oracle_combine(int64_t T, int64_t H, int64_t K, int64_t R,
                    const uint16_t *y, const float *recv_topk_weights,
                    const int32_t *rank_prefix_matrix, const int32_t *send_head,
                    uint16_t *out, float *combined_topk_weights)
{
    float *acc = (float *)malloc((size_t)(H > 0 ? H : 1) * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int64_t r = 0; r < R; ++r) {
            int32_t p = send_head[t * R + r];
            if (p < 0)
                continue;
            int64_t row = (r > 0 ? rank_prefix_matrix[r - 1] : 0) + p;
            for (int64_t h = 0; h < H; ++h)
                acc[h] += bf16_to_f32(y[row * H + h]);
        }
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = f32_to_bf16_rne(acc[h]);

        if (combined_topk_weights != NULL && recv_topk_weights != NULL) {
            for (int64_t k = 0; k < K; ++k) {
                float w = 0.0f;
                for (int64_t r = 0; r < R; ++r) {
                    int32_t p = send_head[t * R + r];
                    if (p < 0)
                        continue;
                    int64_t row = (r > 0 ? rank_prefix_matrix[r - 1] : 0) + p;
                    w += recv_topk_weights[row * K + k];
                }
                combined_topk_weights[t * K + k] = w;
            }
        }
    }
    free(acc);
}

/* ------------------------------------------------------------ low latency --- */

/* Slot of (t, k) inside its expert's receive area: the number of earlier
 * (t', k') pairs, in (token, slot) order, that name the same expert.
 * Reading: the pages leave the order open; token order is taken. */
static void ll_slots(int64_t T, int64_t K, int64_t E, const int64_t *topk_idx, int32_t *slot,
                     int32_t *count)
{
    for (int64_t e = 0; e < E; ++e)
        count[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0 || e >= E) {
                slot[t * K + k] = -1;
                continue;
            }
            slot[t * K + k] = count[e]++;
        }
    }
}

/*
 * Low-latency dispatch, [P1] "IB-GDA Kernels": each (token, slot) pair is
 * streamed straight into its expert's own receive area, with per-expert
 * counts.  Expert e = r*epr + le lives on rank r as local expert le.
 *   buf[le][r][s][:]   = x[t] for the pair (t, k) whose slot is s
 *   counts[le][r]      = number of pairs routed to e
 *   src_info[le][r][s] = t, -1 for unused slots
 *   topk_slot[t][k]    = s, -1 for masked slots or slots past capacity
 * Pairs whose slot is >= num_slots are dropped (reading); counts still report
 * the true number.  Unused buf rows are left untouched.
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_ll_dispatch(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R, int64_t num_slots,
                       const uint16_t *x, const int64_t *topk_idx, uint16_t *buf,
                       int32_t *counts, int32_t *src_info, int32_t *topk_slot)
{
    if (E % R != 0 || num_slots < 1)
        return -1;
    int64_t epr = E / R;
    int32_t *cnt = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    ll_slots(T, K, E, topk_idx, topk_slot, cnt);
    for (int64_t i = 0; i < epr * R * num_slots; ++i)
        src_info[i] = -1;
    for (int64_t e = 0; e < E; ++e)
        counts[(e % epr) * R + e / epr] = cnt[e];
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            int64_t s = topk_slot[t * K + k];
            if (e < 0 || s < 0)
                continue;
            if (s >= num_slots) {
                topk_slot[t * K + k] = -1;
                continue;
            }
            int64_t le = e % epr, r = e / epr;
            int64_t cell = (le * R + r) * num_slots + s;
            src_info[cell] = (int32_t)t;
            if (buf != NULL)
                memcpy(buf + cell * H, x + t * H, (size_t)H * sizeof(uint16_t));
        }
    }
    free(cnt);
    return 0;
}

/*
 * Low-latency combine, [P1] "IB-GDA Kernels": each token gathers the K rows
 * its slots produced and reduces them weighted by its top-k weights:
 *   out[t][h] = bf16_rne( acc ),  acc = fma(w[t][k], f32(buf[cell(t,k)][h]), acc)
 * over k ascending, valid in-capacity slots only, from acc = +0 (reading: the
 * pages give no order; ascending slot with a fused multiply-add is taken).
 * The slots are recomputed here from topk_idx by the definition above.
 */
int oracle_ll_combine(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R, int64_t num_slots,
                      const uint16_t *buf, const int64_t *topk_idx, const float *topk_weights,
                      uint16_t *out)
{
    if (E % R != 0 || num_slots < 1)
        return -1;
    int64_t epr = E / R;
    int32_t *slot = (int32_t *)malloc((size_t)(T * K > 0 ? T * K : 1) * sizeof(int32_t));
    int32_t *cnt = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    float *acc = (float *)malloc((size_t)(H > 0 ? H : 1) * sizeof(float));
    ll_slots(T, K, E, topk_idx, slot, cnt);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            int64_t s = slot[t * K + k];
            if (e < 0 || s < 0 || s >= num_slots)
                continue;
            float w = topk_weights[t * K + k];
            int64_t cell = ((e % epr) * R + e / epr) * num_slots + s;
            for (int64_t h = 0; h < H; ++h)
                acc[h] = fmaf(w, bf16_to_f32(buf[cell * H + h]), acc[h]);
        }
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = f32_to_bf16_rne(acc[h]);
    }
    free(acc);
    free(cnt);
    free(slot);
    return 0;
}

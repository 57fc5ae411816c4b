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
 *   [P5] "Chapter 10, V2: buffers beyond EP" (bowenzhou.top), section 10.2
 *        (lb_prefetch_weights / lb_reduce_grads with a redundancy mapping).
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

/* [P1] "Dynamic Rank Masking": rank r is masked when rank_mask is given and
 * rank_mask[r] is nonzero (1 = masked, 0 = active). */
static int rank_masked(const int32_t *rank_mask, int64_t r)
{
    return rank_mask != NULL && rank_mask[r] != 0;
}

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
 * rank_mask[R] (nullable): reading of "Dynamic Rank Masking" for this path: a
 * slot whose expert lives on a masked rank is treated exactly like a masked
 * slot, so a masked rank receives nothing and its experts count 0.
 * Returns N, or -1 on invalid arguments.
 */
int64_t oracle_layout(int64_t T, int64_t K, int64_t E, int64_t R, int64_t C,
                      const int64_t *topk_idx, const int32_t *rank_mask,
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
            if (rank_masked(rank_mask, e / epr))
                continue; /* expert on a masked rank: as a masked slot */
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
 * Bias terms ([P1] "Combine Operation" names them without a formula):
 * reading: bias0 then bias1, bf16 [T][H] each, nullable, added in fp32 after
 * the rank sum and before the single rounding to bf16.
 * The optional weight output is the same reduction of recv_topk_weights,
 * kept in fp32 (the reduced weights the pages' combine returns).
 * rank_mask[R] (nullable, "Dynamic Rank Masking"): ranks masked at combine
 * time are skipped, as if t had not gone there (rows and weights).
 */
void oracle_combine(int64_t T, int64_t H, int64_t K, int64_t R,
                    const uint16_t *y, const float *recv_topk_weights,
                    const int32_t *rank_prefix_matrix, const int32_t *send_head,
                    const uint16_t *bias0, const uint16_t *bias1, const int32_t *rank_mask,
                    uint16_t *out, float *combined_topk_weights)
{
    float *acc = (float *)malloc((size_t)(H > 0 ? H : 1) * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int64_t r = 0; r < R; ++r) {
            int32_t p = send_head[t * R + r];
            if (rank_masked(rank_mask, r))
                continue;
            if (p < 0)
                continue;
            int64_t row = (r > 0 ? rank_prefix_matrix[r - 1] : 0) + p;
            for (int64_t h = 0; h < H; ++h)
                acc[h] += bf16_to_f32(y[row * H + h]);
        }
        if (bias0 != NULL)
            for (int64_t h = 0; h < H; ++h)
                acc[h] += bf16_to_f32(bias0[t * H + h]);
        if (bias1 != NULL)
            for (int64_t h = 0; h < H; ++h)
                acc[h] += bf16_to_f32(bias1[t * H + h]);
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = f32_to_bf16_rne(acc[h]);

        if (combined_topk_weights != NULL && recv_topk_weights != NULL) {
            for (int64_t k = 0; k < K; ++k) {
                float w = 0.0f;
                for (int64_t r = 0; r < R; ++r) {
                    int32_t p = send_head[t * R + r];
                    if (p < 0 || rank_masked(rank_mask, r))
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

/* Is pair (t, k) sent?  Its slot must be valid, and its expert's rank must
 * not be masked.  [P1] "Dynamic Rank Masking": a masked rank (mask value 1)
 * stops taking part without tearing the context down; reading: its pairs are
 * treated exactly like masked slots (not sent, not counted, not combined).
 * rank_mask may be NULL (no rank masked). */
static int ll_live(int64_t e, int64_t E, int64_t epr, const int32_t *rank_mask)
{
    if (e < 0 || e >= E)
        return 0;
    if (rank_mask != NULL && rank_mask[e / epr] != 0)
        return 0;
    return 1;
}

/* Slot of (t, k) inside its expert's receive area: the number of earlier
 * live (t', k') pairs, in (token, slot) order, that name the same expert.
 * Reading: the pages leave the order open; token order is taken. */
static void ll_slots(int64_t T, int64_t K, int64_t E, int64_t epr, const int32_t *rank_mask,
                     const int64_t *topk_idx, int32_t *slot, int32_t *count)
{
    for (int64_t e = 0; e < E; ++e)
        count[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (!ll_live(e, E, epr, rank_mask)) {
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
                       const uint16_t *x, const int64_t *topk_idx, const int32_t *rank_mask,
                       uint16_t *buf, int32_t *counts, int32_t *src_info, int32_t *topk_slot)
{
    if (E % R != 0 || num_slots < 1)
        return -1;
    int64_t epr = E / R;
    int32_t *cnt = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    ll_slots(T, K, E, epr, rank_mask, topk_idx, topk_slot, cnt);
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
 * The slots are recomputed here from topk_idx by the definition above, with
 * the rank mask the dispatch used (rank_mask).  combine_mask (nullable) masks
 * ranks at combine time: their pairs contribute nothing, whatever the
 * dispatch did (a rank that failed after the dispatch).
 */
int oracle_ll_combine(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R, int64_t num_slots,
                      const uint16_t *buf, const int64_t *topk_idx, const float *topk_weights,
                      const int32_t *rank_mask, const int32_t *combine_mask, uint16_t *out)
{
    if (E % R != 0 || num_slots < 1)
        return -1;
    int64_t epr = E / R;
    int32_t *slot = (int32_t *)malloc((size_t)(T * K > 0 ? T * K : 1) * sizeof(int32_t));
    int32_t *cnt = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    float *acc = (float *)malloc((size_t)(H > 0 ? H : 1) * sizeof(float));
    ll_slots(T, K, E, epr, rank_mask, topk_idx, slot, cnt);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            int64_t s = slot[t * K + k];
            if (e < 0 || s < 0 || s >= num_slots)
                continue;
            if (combine_mask != NULL && combine_mask[e / epr] != 0)
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

/* ------------------------------------------------------------------ FP8 --- */

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, 0x7F / 0xFF are NaN, largest finite 448 = 1.75 * 2^8,
 * smallest normal 2^-6, subnormals m * 2^-9 (m = 1..7). */
float oracle_e4m3_to_f32(uint8_t c)
{
    int sign = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    double v;
    if (ex == 15 && m == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, ex - 7);
    return (float)(sign ? -v : v);
}

/* Round to nearest, ties to even, saturating at +-448 (the finite range is
 * what a scaled activation needs; there is no infinity to round to). */
uint8_t oracle_f32_to_e4m3(float f)
{
    if (isnan(f))
        return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0;
    double a = fabs((double)f);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        double q = rint(a * 512.0); /* units of 2^-9; 8 is the smallest normal */
        return sign | (uint8_t)q;
    }
    int e;
    double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
    e -= 1;                   /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double mi = rint((2.0 * fr - 1.0) * 8.0);
    if (mi == 8.0) {
        mi = 0.0;
        e += 1;
    }
    int code = ((e + 7) << 3) | (int)mi;
    if (code > 0x7E)
        code = 0x7E;
    return sign | (uint8_t)code;
}

void oracle_f32_to_e4m3_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(in[i]);
}

/*
 * Low-latency dispatch with FP8 payload ([P1] "IB-GDA Kernels": FP8 when
 * use_fp8 is set; the pages' code example sets it on the dispatch).  Slots,
 * counts, src_info and topk_slot are those of oracle_ll_dispatch.  Each sent
 * row is cut into blocks of 128 elements; per block (reading, the pages give
 * no recipe):
 *   amax  = max(max |x|, 1e-4)               (fp32)
 *   sinv  = 448 / amax                        (fp32 division)
 *   q[h]  = e4m3_rne_sat(x[h] * sinv)         (fp32 product, then rounding)
 *   scale = amax / 448                        (fp32 division; x ~ q * scale)
 * packed_q [E/R][R][slots][H] bytes, packed_scale [E/R][R][slots][H/128].
 * Requires H % 128 == 0.  Returns 0, or -1 on invalid arguments.
 */
int oracle_ll_dispatch_fp8(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R,
                           int64_t num_slots, const uint16_t *x, const int64_t *topk_idx,
                           const int32_t *rank_mask, uint8_t *packed_q, float *packed_scale,
                           int32_t *counts, int32_t *src_info, int32_t *topk_slot)
{
    if (H % 128 != 0)
        return -1;
    int rc = oracle_ll_dispatch(T, H, K, E, R, num_slots, x, topk_idx, rank_mask, NULL, counts,
                                src_info, topk_slot);
    if (rc != 0)
        return rc;
    int64_t epr = E / R, nb = H / 128;
    for (int64_t cell = 0; cell < epr * R * num_slots; ++cell) {
        int32_t t = src_info[cell];
        if (t < 0)
            continue;
        for (int64_t b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int64_t h = b * 128; h < (b + 1) * 128; ++h) {
                float v = fabsf(bf16_to_f32(x[t * H + h]));
                if (v > amax)
                    amax = v;
            }
            if (amax < 1e-4f)
                amax = 1e-4f;
            float sinv = 448.0f / amax;
            packed_scale[cell * nb + b] = amax / 448.0f;
            for (int64_t h = b * 128; h < (b + 1) * 128; ++h)
                packed_q[cell * H + h] = oracle_f32_to_e4m3(bf16_to_f32(x[t * H + h]) * sinv);
        }
    }
    return 0;
}

/* ------------------------------------------------------- load balancing --- */

/*
 * [P5] 10.2: lb_reduce_grads folds the gradients of redundant expert
 * replicas back into the experts they copy, following redundancy_mapping
 * (replica j copies expert mapping[j]).  Reading: bf16 gradients, fp32
 * accumulation starting from the expert's own gradient, replicas added in
 * ascending j, one rounding to bf16; experts with no replica are untouched;
 * mapping entries outside [0, E) are ignored.
 *   expert_grads [E][P] (in/out), redundant_grads [n_rep][P].
 */
void oracle_lb_reduce_grads(int64_t n_rep, int64_t E, int64_t P, const uint16_t *redundant_grads,
                            uint16_t *expert_grads, const int64_t *mapping)
{
    float *acc = (float *)malloc((size_t)(P > 0 ? P : 1) * sizeof(float));
    for (int64_t e = 0; e < E; ++e) {
        int any = 0;
        for (int64_t j = 0; j < n_rep; ++j)
            any |= mapping[j] == e;
        if (!any)
            continue;
        for (int64_t p = 0; p < P; ++p)
            acc[p] = bf16_to_f32(expert_grads[e * P + p]);
        for (int64_t j = 0; j < n_rep; ++j)
            if (mapping[j] == e)
                for (int64_t p = 0; p < P; ++p)
                    acc[p] += bf16_to_f32(redundant_grads[j * P + p]);
        for (int64_t p = 0; p < P; ++p)
            expert_grads[e * P + p] = f32_to_bf16_rne(acc[p]);
    }
    free(acc);
}

/*
 * Low-latency combine of an FP8 payload ([P1] "IB-GDA Kernels": FP8 with
 * use_fp8; reading: the codes and per-128-element-block scales of
 * oracle_ll_dispatch_fp8 are decoded in the combine).  Each element of a
 * cell is decoded exactly to fp32 and multiplied by its block's scale in
 * fp32 (one rounding); the weighted sum then runs exactly as in
 * oracle_ll_combine: fmaf over k ascending from +0, one RNE to bf16.
 *   q     [epr][R][num_slots][H] e4m3 codes
 *   scale [epr][R][num_slots][H/128] fp32
 */
int oracle_ll_combine_fp8(int64_t T, int64_t H, int64_t K, int64_t E, int64_t R,
                          int64_t num_slots, const uint8_t *q, const float *scale,
                          const int64_t *topk_idx, const float *topk_weights,
                          const int32_t *rank_mask, const int32_t *combine_mask, uint16_t *out)
{
    if (E % R != 0 || num_slots < 1 || H % 128 != 0)
        return -1;
    int64_t epr = E / R, nb = H / 128;
    int32_t *slot = (int32_t *)malloc((size_t)(T * K > 0 ? T * K : 1) * sizeof(int32_t));
    int32_t *cnt = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    float *acc = (float *)malloc((size_t)(H > 0 ? H : 1) * sizeof(float));
    ll_slots(T, K, E, epr, rank_mask, topk_idx, slot, cnt);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            int64_t s = slot[t * K + k];
            if (e < 0 || s < 0 || s >= num_slots)
                continue;
            if (combine_mask != NULL && combine_mask[e / epr] != 0)
                continue;
            float w = topk_weights[t * K + k];
            int64_t cell = ((e % epr) * R + e / epr) * num_slots + s;
            for (int64_t h = 0; h < H; ++h) {
                float v = oracle_e4m3_to_f32(q[cell * H + h]) * scale[cell * nb + h / 128];
                acc[h] = fmaf(w, v, acc[h]);
            }
        }
        for (int64_t h = 0; h < H; ++h)
            out[t * H + h] = f32_to_bf16_rne(acc[h]);
    }
    free(acc);
    free(cnt);
    free(slot);
    return 0;
}

/* [P5] 10.2: lb_prefetch_weights copies each expert's weights into its
 * replicas' slots before the expert computation: redundant[j] =
 * expert[mapping[j]]; replicas with an invalid mapping entry are untouched. */
void oracle_lb_prefetch_weights(int64_t n_rep, int64_t E, int64_t P, const uint16_t *expert_weights,
                                uint16_t *redundant_weights, const int64_t *mapping)
{
    for (int64_t j = 0; j < n_rep; ++j) {
        int64_t e = mapping[j];
        if (e < 0 || e >= E)
            continue;
        memcpy(redundant_weights + j * P, expert_weights + e * P, (size_t)P * sizeof(uint16_t));
    }
}

// combine.hip -- combine gather-reduce on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "Combine Operation": the rows a token sent out come back and are reduced by
// addition into that token's position, using the dispatch handle to find
// them.  Here the rows of token t sit at S[r] + send_head[t][r] in one buffer;
// a group of G lanes (whole wavefronts) reads them in ascending rank order
// (the layout's per-token row list is already in that order), adds them in
// fp32 registers starting from +0, and writes one bf16 row rounded to
// nearest even.  The optional weight reduction sums the per-row top-k
// weights the same way.
//
// The optional bias terms of the same section (reading: one or two bf16
// [T][H] tensors) are added in fp32 after the rank sum, bias0 then bias1,
// before the single rounding.
//
// A rank mask given at combine time ("Dynamic Rank Masking": nonzero =
// masked) drops that rank's rows and weights: the wavefront moves the live
// entries of the row list to its front (a bijective lane permute) before
// the sum, keeping their ascending order.
//
// The sum order is fixed (rank ascending, one add per row per element), so the
// result does not depend on the launch shape.  U rows' loads are issued
// before any of them is added, so each lane keeps U*VPT 16-byte loads in
// flight; the row list is loaded once per wavefront and broadcast with
// readlane (no LDS, no barrier).

#include <atomic>
#include <cstdio>
#include <cstdlib>

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kCombineBlock = 256;

template <int VPT>
__device__ __forceinline__ void add_row(float (&acc)[VPT][8], const u32x4 (&v)[VPT])
{
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[i][2 * q] += bf16_lo(v[i][q]);
            acc[i][2 * q + 1] += bf16_hi(v[i][q]);
        }
    }
}

template <bool NTL>
__device__ __forceinline__ u32x4 load_row_vec(const u32x4 *p)
{
    if (NTL)
        return __builtin_nontemporal_load(p);
    return *p;
}

// A group of G lanes reduces one slice of one token's row at a time: the
// row's chunks of G*VPT vectors are dealt round-robin to S groups (S = 1: one
// group per token).  With a persistent grid (fewer groups than token slices)
// each group walks them with a grid stride.  NTL: rows are loaded
// nontemporally (each is read exactly once).  The slice-0 group reduces the
// weights.
template <int G, int VPT, int U, bool NTL, bool kBias>
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(
    const u32x4 *__restrict__ y, int T, int V, int K, int kmax, int S,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int32_t *__restrict__ rank_mask, const float *__restrict__ recv_topk_weights,
    const u32x4 *__restrict__ bias0, const u32x4 *__restrict__ bias1,
    u32x4 *__restrict__ out, float *__restrict__ combined_topk_weights)
{
    constexpr int kGroups = kCombineBlock / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gt = threadIdx.x % G;
    const int first = __builtin_amdgcn_readfirstlane(blockIdx.x * kGroups + threadIdx.x / G);
    const int stride = gridDim.x * kGroups;
    for (int ts = first; ts < T * S; ts += stride) {
        const int t = ts / S;
        const int slice = ts - t * S;
        int rowv = lane < kmax ? dst_row[int64_t(t) * kmax + lane] : -1;
        if (rank_mask != nullptr) {
            const int rk = rowv >= 0 ? dst_rank[int64_t(t) * kmax + lane] : 0;
            const bool live = rowv >= 0 && rank_mask[rk] == 0;
            const uint64_t lm = wave_ballot(live);
            const uint64_t below = lanemask_lt();
            const int nl = __popcll(lm);
            const int to = live ? __popcll(lm & below) : nl + __popcll(~lm & below);
            rowv = __builtin_amdgcn_ds_permute(to << 2, live ? rowv : -1);
        }
        const int nhit = __popcll(wave_ballot(rowv >= 0));

        for (int base = slice * G * VPT; base < V; base += S * G * VPT) {
            float acc[VPT][8];
#pragma unroll
            for (int i = 0; i < VPT; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[i][q] = 0.0f;

            for (int j = 0; j < nhit; j += U) {
                u32x4 v[U][VPT];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool live = j + u < nhit;
                    const int row = __builtin_amdgcn_readlane(rowv, live ? j + u : 0);
                    const u32x4 *yr = y + int64_t(row) * V;
#pragma unroll
                    for (int i = 0; i < VPT; ++i) {
                        const int idx = base + i * G + gt;
                        v[u][i] = (live && idx < V) ? load_row_vec<NTL>(yr + idx)
                                                    : u32x4{0, 0, 0, 0};
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (j + u < nhit)
                        add_row<VPT>(acc, v[u]);
            }
            // Bias terms: after the rank sum, before the one rounding.
            const u32x4 *biases[2] = {bias0, bias1};
            for (int bi = 0; kBias && bi < 2; ++bi) {
                const u32x4 *bias = biases[bi];
                if (bias == nullptr)
                    continue;
                u32x4 bv[VPT];
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int idx = base + i * G + gt;
                    bv[i] = idx < V ? bias[int64_t(t) * V + idx] : u32x4{0, 0, 0, 0};
                }
                add_row<VPT>(acc, bv);
            }

            u32x4 *o = out + int64_t(t) * V;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * G + gt;
                if (idx < V) {
                    u32x4 r;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        r[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
                    __builtin_nontemporal_store(r, o + idx);
                }
            }
        }

        if (combined_topk_weights != nullptr && slice == 0) {
            // up to 8 rows' weights loaded at once, then added in rank order
            constexpr int kW = 8;
            for (int k = gt; k < K; k += G) {
                float w = 0.0f;
                for (int j0 = 0; j0 < nhit; j0 += kW) {
                    float wv[kW];
#pragma unroll
                    for (int u = 0; u < kW; ++u) {
                        const int j = j0 + u < nhit ? j0 + u : 0;
                        const int64_t row = __builtin_amdgcn_readlane(rowv, j);
                        wv[u] = recv_topk_weights[row * K + k];
                    }
#pragma unroll
                    for (int u = 0; u < kW; ++u)
                        if (j0 + u < nhit)
                            w += wv[u];
                }
                combined_topk_weights[int64_t(t) * K + k] = w;
            }
        }
    }
}

// Gather form (a tuning shape): workgroup (t, yb) sums chunk yb (BT vectors)
// of token t's rows, one thread per 16-byte vector: the token's rows are
// taken kGatherRows at a time, all their loads in flight before any is added,
// in ascending rank from +0 as above (rows on a rank masked now skipped, so
// the order of the rest is kept), then the biases, then one rounding.  One
// load per row and thread, in many short workgroups.  Unweighted, right after
// a dispatch, it took 87.6 against 91.6 us at the training-scale batch; in
// the whole step, weighted, it measured the same as the token-major form.
// The chunk-0 workgroup's lanes k < K also sum weight k of the same rows.
constexpr int kGatherRows = 8;

template <int BT, bool kBias>
__global__ __launch_bounds__(BT) void combine_gather_kernel(
    const u32x4 *__restrict__ y, int T, int V, int K, int kmax, int ny,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int32_t *__restrict__ rank_mask, const float *__restrict__ recv_topk_weights,
    const u32x4 *__restrict__ bias0, const u32x4 *__restrict__ bias1,
    u32x4 *__restrict__ out, float *__restrict__ combined_topk_weights)
{
    const int64_t t = blockIdx.x / ny;
    const int yb = int(blockIdx.x - t * ny);
    const int tid = threadIdx.x;
    const int c = yb * BT + tid;
    const int cc = c < V ? c : V - 1;  // lanes past the row re-read its last vector (not stored)
    const int32_t *rl = dst_row + t * kmax;
    // chunk 0's lanes k < K also sum weight k of the same rows (K <= 64 < BT)
    const bool wsum = combined_topk_weights != nullptr && yb == 0 && tid < K;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        acc[q] = 0.0f;
    float w = 0.0f;
    // a token with no rows loads nothing (y may then hold no rows at all);
    // rows past the list or on masked ranks re-read the token's first row
    const int row0 = rl[0];
    bool more = row0 >= 0;
    for (int k0 = 0; more && k0 < kmax; k0 += kGatherRows) {
        int row[kGatherRows];
#pragma unroll
        for (int j = 0; j < kGatherRows; ++j) {
            const int k = k0 + j;
            row[j] = k < kmax ? rl[k] : -1;  // rows are packed first, then -1
            if (row[j] >= 0 && rank_mask != nullptr && rank_mask[dst_rank[t * kmax + k]] != 0)
                row[j] = -2;  // on a rank masked now: skipped, the list goes on
        }
        u32x4 v[kGatherRows];
        float wv[kGatherRows];
#pragma unroll
        for (int j = 0; j < kGatherRows; ++j) {
            const int64_t r = row[j] >= 0 ? row[j] : row0;
            v[j] = load_row_vec<true>(y + r * V + cc);
            wv[j] = wsum ? recv_topk_weights[r * K + tid] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kGatherRows; ++j) {
            if (row[j] == -1) {
                more = false;
                break;
            }
            if (row[j] < 0)
                continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo(v[j][q]);
                acc[2 * q + 1] += bf16_hi(v[j][q]);
            }
            w += wv[j];
        }
    }
    if (kBias) {
        // after the rank sum, before the one rounding: bias0, then bias1
        const u32x4 *biases[2] = {bias0, bias1};
        for (int bi = 0; bi < 2; ++bi) {
            if (biases[bi] == nullptr)
                continue;
            const u32x4 bv = biases[bi][t * V + cc];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo(bv[q]);
                acc[2 * q + 1] += bf16_hi(bv[q]);
            }
        }
    }
    if (c < V) {
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        __builtin_nontemporal_store(r, out + t * V + c);
    }
    if (wsum)
        combined_topk_weights[t * K + tid] = w;
}

// The two kernels share one argument list; the gather kernel takes its
// chunk count ny where the token-major kernel takes S.
typedef void (*CombineFn)(const u32x4 *, int, int, int, int, int, const int32_t *,
                          const int32_t *, const int32_t *, const float *, const u32x4 *,
                          const u32x4 *, u32x4 *, float *);

// A launch shape.  Token-major: G lanes per group, VPT vectors per lane, S
// groups per token (row slices), U rows in flight, NTL nontemporal row
// loads, and P = persistent block count (0: one group per token slice).
// Gather: G threads per workgroup, one vector each, kGatherRows rows in
// flight, nontemporal loads.  The tuning knob addresses shapes as (G, VPT,
// X*10000 + S*1000 + U*100 + NTL*10 + P/256), X = 1 for the gather form.
struct CombineCfg {
    int G, VPT, S, U, NTL, P;
    CombineFn fn, fn_bias;
    int gather;
};

#define EP_COMBINE_CFG(G, VPT, S, U, NTL, P)                                               \
    {G, VPT, S, U, NTL, P, combine_kernel<G, VPT, U, NTL, false>,                          \
     combine_kernel<G, VPT, U, NTL, true>, 0}
#define EP_GATHER_CFG(BT)                                                                    \
    {BT, 1, 1, kGatherRows, 1, 0, combine_gather_kernel<BT, false>,                          \
     combine_gather_kernel<BT, true>, 1}

const CombineCfg kCombineCfgs[] = {
    EP_COMBINE_CFG(256, 1, 1, 2, 1, 0), EP_COMBINE_CFG(256, 2, 1, 2, 1, 0),
    EP_COMBINE_CFG(256, 4, 1, 2, 1, 0), EP_COMBINE_CFG(256, 4, 1, 4, 1, 0),
    EP_COMBINE_CFG(128, 7, 1, 1, 1, 0), EP_COMBINE_CFG(128, 7, 1, 1, 0, 0),
    EP_COMBINE_CFG(128, 7, 1, 2, 1, 0), EP_COMBINE_CFG(128, 8, 1, 2, 1, 0),
    EP_COMBINE_CFG(64, 14, 1, 1, 1, 0), EP_COMBINE_CFG(64, 7, 2, 1, 1, 0),
    EP_COMBINE_CFG(64, 7, 2, 2, 1, 0),  EP_COMBINE_CFG(64, 4, 4, 2, 1, 0),
    EP_COMBINE_CFG(64, 2, 7, 4, 1, 0),  EP_COMBINE_CFG(64, 2, 7, 8, 1, 0),
    EP_COMBINE_CFG(64, 1, 14, 8, 1, 0),
    EP_GATHER_CFG(448), EP_GATHER_CFG(128),
};

int combine_code(const CombineCfg &c)
{
    return c.gather * 10000 + c.S * 1000 + c.U * 100 + c.NTL * 10 + c.P / 256;
}

std::atomic<int> g_over_g{-2}, g_over_v{-1}, g_over_u{-1};  // -2: env not read yet

// Launch shape for rows of V vectors.  An override (ep_set_tuning, or the env
// var EP_TUNE_COMBINE="G,VPT,U") wins; results never depend on it.
// Otherwise: one chunk that covers the row exactly, one row in flight,
// nontemporal row loads (measured best on the training-scale rows: the rows
// are read once, and keeping them out of the caches leaves the caches to the
// data that is reused).  The gather form measured the same in the step
// (92.0-93.0 against 92.8-93.1 us, one box), so the token-major form stays.
const CombineCfg &pick(int V)
{
    if (g_over_g.load() == -2) {
        int g = -1, v = -1, u = -1;
        if (const char *s = std::getenv("EP_TUNE_COMBINE"))
            if (std::sscanf(s, "%d,%d,%d", &g, &v, &u) != 3)
                g = v = u = -1;
        g_over_v = v;
        g_over_u = u;
        g_over_g = g;
    }
    const int og = g_over_g.load(), ov = g_over_v.load(), ou = g_over_u.load();
    for (const CombineCfg &c : kCombineCfgs)
        if (c.G == og && c.VPT == ov && combine_code(c) == ou)
            return c;
    for (const CombineCfg &c : kCombineCfgs)
        if (!c.gather && c.S == 1 && c.U == 1 && c.NTL == 1 && c.P == 0 && c.G * c.VPT == V &&
            c.G >= 128)
            return c;
    if (V <= 256)
        return kCombineCfgs[0];
    if (V <= 512)
        return kCombineCfgs[1];
    return kCombineCfgs[2];
}

}  // namespace

bool set_combine_tuning(int g, int vpt, int u)
{
    if (g == -1 && vpt == -1 && u == -1) {
        g_over_v = -1;
        g_over_u = -1;
        g_over_g = -1;
        return true;
    }
    for (const CombineCfg &c : kCombineCfgs)
        if (c.G == g && c.VPT == vpt && combine_code(c) == u) {
            g_over_v = vpt;
            g_over_u = u;
            g_over_g = g;
            return true;
        }
    return false;
}

int combine_tuning_count() { return int(sizeof(kCombineCfgs) / sizeof(kCombineCfgs[0])); }

void combine_tuning_at(int i, int *g, int *vpt, int *u)
{
    *g = kCombineCfgs[i].G;
    *vpt = kCombineCfgs[i].VPT;
    *u = combine_code(kCombineCfgs[i]);
}

hipError_t launch_combine(const LayoutShape &s, int hidden, const void *y, const LayoutBufs &b,
                          const float *recv_topk_weights, const void *bias0, const void *bias1,
                          const int32_t *rank_mask, void *out, float *combined_topk_weights,
                          hipStream_t stream)
{
    if (s.T == 0)
        return hipSuccess;
    const int V = hidden / 8;
    const CombineCfg &c = pick(V);
    const bool bias = bias0 != nullptr || bias1 != nullptr;
    if (c.gather) {
        const int ny = (V + c.G - 1) / c.G;
        const int64_t blocks = int64_t(s.T) * ny;
        if (log_enabled())
            log_launch("combine_gather T=%d H=%d K=%d R=%d: BT=%d chunks=%d blocks=%lld%s%s",
                       s.T, hidden, s.K, s.R, c.G, ny, (long long)blocks, bias ? " +bias" : "",
                       rank_mask != nullptr ? " +mask" : "");
        hipLaunchKernelGGL(bias ? c.fn_bias : c.fn, dim3(unsigned(blocks)), dim3(c.G), 0, stream,
                           static_cast<const u32x4 *>(y), s.T, V, s.K, s.kmax, ny, b.dst_row,
                           b.dst_rank, rank_mask, recv_topk_weights,
                           static_cast<const u32x4 *>(bias0), static_cast<const u32x4 *>(bias1),
                           static_cast<u32x4 *>(out), combined_topk_weights);
        return hipGetLastError();
    }
    const int per_block = kCombineBlock / c.G;
    const int64_t groups = int64_t(s.T) * c.S;
    int blocks = int((groups + per_block - 1) / per_block);
    if (c.P > 0 && c.P < blocks)
        blocks = c.P;
    if (log_enabled())
        log_launch("combine T=%d H=%d K=%d R=%d: G=%d VPT=%d S=%d U=%d NTL=%d blocks=%d%s%s", s.T,
                   hidden, s.K, s.R, c.G, c.VPT, c.S, c.U, c.NTL, blocks, bias ? " +bias" : "",
                   rank_mask != nullptr ? " +mask" : "");
    hipLaunchKernelGGL(bias ? c.fn_bias : c.fn, dim3(blocks), dim3(kCombineBlock), 0, stream,
                       static_cast<const u32x4 *>(y), s.T, V, s.K, s.kmax, c.S, b.dst_row,
                       b.dst_rank, rank_mask, recv_topk_weights, static_cast<const u32x4 *>(bias0),
                       static_cast<const u32x4 *>(bias1), static_cast<u32x4 *>(out),
                       combined_topk_weights);
    return hipGetLastError();
}

}  // namespace ep

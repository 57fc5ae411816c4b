// dispatch.hip -- dispatch pack on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "Dispatch Operation": every token row is sent once to each rank that hosts
// one of its experts, with the token's expert ids (renumbered local to the
// receiving rank) and weights.  Here the R ranks are R contiguous segments of
// one buffer, so the all-to-all becomes a gather-scatter copy: row
// S[r] + send_head[t][r] receives x[t].  The same kernel without the top-k
// outputs is the handle-reuse fast path of "How DeepEP Optimizes Handle
// Reuse for Repeated Dispatches" ("Fast Path Dispatch with Handle Reuse").
//
// Token-major: a group of G lanes (one or more whole wavefronts) owns one
// token.  It reads the token's row from HBM once into VGPRs (VPT 16-byte
// vectors per lane, fully coalesced) and stores it to each destination row
// (at most min(K, R), from the layout's per-token row list, which every
// wavefront loads once and broadcasts with readlane -- no LDS, no barrier).
// Reading x once keeps the kernel at the algorithmic byte count whatever the
// segment sizes; skewed routing only changes how many stores a group issues.
// Stores are nontemporal: packed rows are not re-read by this kernel and
// should not evict the rows still to be read.

#include <atomic>
#include <cstdio>
#include <cstdlib>

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kPackBlock = 256;

template <bool NTS>
__device__ __forceinline__ void store_row_vec(u32x4 v, u32x4 *p)
{
    if (NTS)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <bool NTL>
__device__ __forceinline__ u32x4 load_x_vec(const u32x4 *p)
{
    if (NTL)
        return __builtin_nontemporal_load(p);
    return *p;
}

// A group of G lanes packs one slice of one token's row at a time: the row's
// chunks of G*VPT vectors are dealt round-robin to S groups (S = 1: one group
// per token), so more, shorter-lived wavefronts share the stores.  With a
// persistent grid (fewer groups than token slices) each group walks them with
// a grid stride.  NTS / NTL: packed rows are stored / token rows loaded
// nontemporally.  The slice-0 group writes the top-k outputs.
template <int G, int VPT, bool NTS, bool NTL, bool kTopk>
__global__ __launch_bounds__(kPackBlock) void dispatch_pack_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int epr, int kmax, int S,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    u32x4 *__restrict__ recv_x, int64_t *__restrict__ recv_topk_idx,
    float *__restrict__ recv_topk_weights)
{
    constexpr int kGroups = kPackBlock / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gt = threadIdx.x % G;
    const int first = __builtin_amdgcn_readfirstlane(blockIdx.x * kGroups + threadIdx.x / G);
    const int stride = gridDim.x * kGroups;
    for (int ts = first; ts < T * S; ts += stride) {
        const int t = ts / S;
        const int slice = ts - t * S;
        const u32x4 *src = x + int64_t(t) * V;
        const int rowv = lane < kmax ? dst_row[int64_t(t) * kmax + lane] : -1;
        const int nhit = __popcll(wave_ballot(rowv >= 0));  // rows are packed first

        if (recv_x != nullptr) {
            for (int base = slice * G * VPT; base < V; base += S * G * VPT) {
                u32x4 v[VPT];
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int idx = base + i * G + gt;
                    if (idx < V)
                        v[i] = load_x_vec<NTL>(src + idx);
                }
                for (int j = 0; j < nhit; ++j) {
                    const int row = __builtin_amdgcn_readlane(rowv, j);
                    u32x4 *dst = recv_x + int64_t(row) * V;
#pragma unroll
                    for (int i = 0; i < VPT; ++i) {
                        const int idx = base + i * G + gt;
                        if (idx < V)
                            store_row_vec<NTS>(v[i], dst + idx);
                    }
                }
            }
        }

        if (kTopk && slice == 0) {
            const int rankv = lane < kmax ? dst_rank[int64_t(t) * kmax + lane] : -1;
            for (int k = gt; k < K; k += G) {
                const int64_t e = topk_idx[int64_t(t) * K + k];
                const float w =
                    recv_topk_weights != nullptr ? topk_weights[int64_t(t) * K + k] : 0.0f;
                const bool valid = e >= 0 && e < E;
                const int er = valid ? int(e) / epr : -1;
                for (int j = 0; j < nhit; ++j) {
                    const int64_t row = __builtin_amdgcn_readlane(rowv, j);
                    const int r = __builtin_amdgcn_readlane(rankv, j);
                    const bool mine = er == r;
                    if (recv_topk_idx != nullptr)
                        recv_topk_idx[row * K + k] = mine ? e - int64_t(r) * epr : -1;
                    if (recv_topk_weights != nullptr)
                        recv_topk_weights[row * K + k] = mine ? w : 0.0f;
                }
            }
        }
    }
}

typedef void (*PackFn)(const u32x4 *, int, int, int, int, int, int, int, const int32_t *,
                       const int32_t *, const int64_t *, const float *, u32x4 *, int64_t *,
                       float *);

// A launch shape: G lanes per group, VPT vectors per lane, S groups per token
// (row slices), NTS / NTL nontemporal stores / loads, P persistent block
// count (0: one group per token slice).  The tuning knob addresses shapes as
// (G, VPT, S*1000 + NTL*100 + NTS*10 + P/256).
struct PackCfg {
    int G, VPT, S, NTS, NTL, P;
    PackFn plain, topk;
};

#define EP_PACK_CFG(G, VPT, S, NTS, NTL, P)                                                \
    {G, VPT, S, NTS, NTL, P, dispatch_pack_kernel<G, VPT, NTS, NTL, false>,                \
     dispatch_pack_kernel<G, VPT, NTS, NTL, true>}

const PackCfg kPackCfgs[] = {
    EP_PACK_CFG(256, 1, 1, 1, 0, 0),  EP_PACK_CFG(256, 2, 1, 1, 0, 0),
    EP_PACK_CFG(256, 4, 1, 1, 0, 0),  EP_PACK_CFG(128, 4, 1, 1, 0, 0),
    EP_PACK_CFG(128, 7, 1, 1, 0, 0),  EP_PACK_CFG(128, 7, 1, 0, 0, 0),
    EP_PACK_CFG(128, 7, 1, 1, 1, 0),  EP_PACK_CFG(128, 8, 1, 1, 0, 0),
    EP_PACK_CFG(64, 14, 1, 1, 0, 0),  EP_PACK_CFG(64, 7, 2, 1, 0, 0),
    EP_PACK_CFG(64, 4, 4, 1, 0, 0),   EP_PACK_CFG(64, 2, 7, 1, 0, 0),
    EP_PACK_CFG(64, 1, 14, 1, 0, 0),  EP_PACK_CFG(64, 2, 7, 0, 0, 0),
    EP_PACK_CFG(64, 2, 7, 1, 0, 1024),
};

int pack_code(const PackCfg &c)
{
    return c.S * 1000 + c.NTL * 100 + c.NTS * 10 + c.P / 256;
}

std::atomic<int> g_over_g{-2}, g_over_v{-1}, g_over_c{-1};  // -2: env not read yet

// Launch shape for a row of V vectors.  An override (ep_set_tuning, or the
// env var EP_TUNE_DISPATCH="G,VPT,code") wins; results never depend on it.
// Otherwise: one chunk that covers the row exactly, with the most lanes,
// nontemporal stores, one group per token.
const PackCfg &pick(int V)
{
    if (g_over_g.load() == -2) {
        int g = -1, v = -1, c = -1;
        if (const char *s = std::getenv("EP_TUNE_DISPATCH"))
            if (std::sscanf(s, "%d,%d,%d", &g, &v, &c) != 3)
                g = v = c = -1;
        g_over_v = v;
        g_over_c = c;
        g_over_g = g;
    }
    const int og = g_over_g.load(), ov = g_over_v.load(), oc = g_over_c.load();
    for (const PackCfg &c : kPackCfgs)
        if (c.G == og && c.VPT == ov && pack_code(c) == oc)
            return c;
    for (int G : {128, 256, 64})
        for (const PackCfg &c : kPackCfgs)
            if (c.G == G && c.G * c.VPT == V && c.S == 1 && c.NTS == 1 && c.NTL == 0 && c.P == 0)
                return c;
    if (V <= 256)
        return kPackCfgs[0];
    if (V <= 512)
        return kPackCfgs[1];
    return kPackCfgs[2];
}

}  // namespace

bool set_dispatch_tuning(int g, int vpt, int code)
{
    if (g == -1 && vpt == -1 && code == -1) {
        g_over_v = -1;
        g_over_c = -1;
        g_over_g = -1;
        return true;
    }
    for (const PackCfg &c : kPackCfgs)
        if (c.G == g && c.VPT == vpt && pack_code(c) == code) {
            g_over_v = vpt;
            g_over_c = code;
            g_over_g = g;
            return true;
        }
    return false;
}

int dispatch_tuning_count() { return int(sizeof(kPackCfgs) / sizeof(kPackCfgs[0])); }

void dispatch_tuning_at(int i, int *g, int *vpt, int *code)
{
    *g = kPackCfgs[i].G;
    *vpt = kPackCfgs[i].VPT;
    *code = pack_code(kPackCfgs[i]);
}

hipError_t launch_dispatch(const LayoutShape &s, int hidden, const void *x, const LayoutBufs &b,
                           const int64_t *topk_idx, const float *topk_weights, void *recv_x,
                           int64_t *recv_topk_idx, float *recv_topk_weights, hipStream_t stream)
{
    if (s.T == 0)
        return hipSuccess;
    const int V = hidden / 8;
    const PackCfg &c = pick(V);
    const bool topk = recv_topk_idx != nullptr || recv_topk_weights != nullptr;
    const int per_block = kPackBlock / c.G;
    const int64_t groups = int64_t(s.T) * c.S;
    int blocks = int((groups + per_block - 1) / per_block);
    if (c.P > 0 && c.P < blocks)
        blocks = c.P;
    if (log_enabled())
        log_launch("dispatch_pack T=%d H=%d K=%d R=%d: G=%d VPT=%d S=%d NTS=%d NTL=%d blocks=%d%s",
                   s.T, hidden, s.K, s.R, c.G, c.VPT, c.S, c.NTS, c.NTL, blocks,
                   topk ? " +topk" : "");
    hipLaunchKernelGGL(topk ? c.topk : c.plain, dim3(blocks), dim3(kPackBlock), 0, stream,
                       static_cast<const u32x4 *>(x), s.T, V, s.K, s.E, s.epr, s.kmax, c.S,
                       b.dst_row,
                       b.dst_rank, topk_idx, topk_weights, static_cast<u32x4 *>(recv_x),
                       recv_topk_idx, recv_topk_weights);
    return hipGetLastError();
}

}  // namespace ep

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
// Two kernels give the same rows.  dispatch_scatter_kernel (the default) is
// destination-major: one thread per 16-byte vector of a few destination
// rows, with workgroups dealt to XCDs so that each token row is read from
// HBM once and re-read from L2 (see the kernel).  The token-major kernel
// below stays as a set of tuning shapes and as the fallback for grids too
// large for the first.
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

// One pass of a group over the chunk [base, base + G*VPT) of a token's row:
// VPT loads, all issued before the row list is consulted (rowv's own load
// was issued earlier; only its ballot waits for it), then the chunk is
// stored to each of the token's nhit destination rows.  Loads past the end
// of the row read its last vector again (in bounds, never stored), so no
// load sits behind a branch.
template <int G, int VPT, bool NTS, bool NTL>
__device__ __forceinline__ void pack_pass(const u32x4 *__restrict__ src, u32x4 *__restrict__ recv_x,
                                          int V, int base, int gt, int rowv)
{
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int idx = base + i * G + gt;
        v[i] = load_x_vec<NTL>(src + (idx < V ? idx : V - 1));
    }
    // The loaded vectors feed only the stores below, which run nhit times;
    // without this the compiler moves the loads under "nhit > 0", i.e.
    // behind the wait for the row list.  Empty and volatile, it keeps them
    // here, all in flight together with the row list's load.
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        asm volatile("" : "+v"(v[i]));
    asm volatile("" : "+v"(rowv));  // (nor may the row list's test move above them)
    const int nhit = __popcll(wave_ballot(rowv >= 0));  // rows are packed first
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

// A group of G lanes packs one slice of one token's row at a time: the row's
// chunks of G*VPT vectors are dealt round-robin to S groups (S = 1: one group
// per token), so more, shorter-lived wavefronts share the stores.  With a
// persistent grid (fewer groups than token slices) each group walks them with
// a grid stride.  NTS / NTL: packed rows are stored / token rows loaded
// nontemporally.  The slice-0 group writes the top-k outputs.  A row that
// one chunk covers (the usual shape: 7168 = 128 lanes x 7 vectors x 8) takes
// a loop-free path, so that the compiler need not wait for the previous
// chunk's stores before it issues the loads.
template <int G, int VPT, bool NTS, bool NTL, bool kTopk>
__global__ __launch_bounds__(kPackBlock) void dispatch_pack_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int epr, int kmax, int S,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    u32x4 *__restrict__ recv_x, int64_t *__restrict__ recv_topk_idx,
    float *__restrict__ recv_topk_weights, const int32_t *__restrict__, const int32_t *__restrict__,
    int, int)
{
    constexpr int kGroups = kPackBlock / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gt = threadIdx.x % G;
    const int first = __builtin_amdgcn_readfirstlane(blockIdx.x * kGroups + threadIdx.x / G);
    const int stride = gridDim.x * kGroups;
    const bool one_pass = S == 1 && V <= G * VPT;
    auto slice_work = [&](int ts) {
        const int t = ts / S;
        const int slice = ts - t * S;
        const u32x4 *src = x + int64_t(t) * V;
        const int rowv = lane < kmax ? dst_row[int64_t(t) * kmax + lane] : -1;
        // The top-k inputs of the slice-0 group are loaded up front, so that
        // their latency overlaps the row's (K <= 64 <= G: one slot per lane).
        const bool topk = kTopk && slice == 0;
        int rankv = -1;
        int64_t e = -1;
        float w = 0.0f;
        if (topk) {
            rankv = lane < kmax ? dst_rank[int64_t(t) * kmax + lane] : -1;
            if (gt < K) {
                e = topk_idx[int64_t(t) * K + gt];
                if (recv_topk_weights != nullptr)
                    w = topk_weights[int64_t(t) * K + gt];
            }
        }

        if (recv_x != nullptr) {
            if (one_pass)
                pack_pass<G, VPT, NTS, NTL>(src, recv_x, V, 0, gt, rowv);
            else
                for (int base = slice * G * VPT; base < V; base += S * G * VPT)
                    pack_pass<G, VPT, NTS, NTL>(src, recv_x, V, base, gt, rowv);
        }

        if (topk) {
            // (their uses stay here: hoisted above the row's loads, they
            // would make those wait for the top-k loads)
            asm volatile("" : "+v"(e), "+v"(w), "+v"(rankv));
            const int nhit = __popcll(wave_ballot(rowv >= 0));
            if (gt < K) {
                const bool valid = e >= 0 && e < E;
                const int er = valid ? int(e) / epr : -1;
                for (int j = 0; j < nhit; ++j) {
                    const int64_t row = __builtin_amdgcn_readlane(rowv, j);
                    const int r = __builtin_amdgcn_readlane(rankv, j);
                    const bool mine = er == r;
                    if (recv_topk_idx != nullptr)
                        recv_topk_idx[row * K + gt] = mine ? e - int64_t(r) * epr : -1;
                    if (recv_topk_weights != nullptr)
                        recv_topk_weights[row * K + gt] = mine ? w : 0.0f;
                }
            }
        }
    };
    if (stride >= T * S) {
        // one token slice per group (the usual launch): no loop around the
        // slice, so nothing makes its loads wait for earlier stores
        if (first < T * S)
            slice_work(first);
    } else {
        for (int ts = first; ts < T * S; ts += stride)
            slice_work(ts);
    }
}

// Destination-major, XCD-grouped (the default): workgroup b writes one
// chunk of BT vectors of kDestGroup destination rows
// of one token -- token t, destinations [kDestGroup*g, kDestGroup*(g+1)) of
// its kmax slots (slots past the token's row count are skipped), chunk yb of
// ny.  The hardware deals workgroup b to XCD b mod 8, and token t's
// workgroups are the b = t (mod 8) ones, consecutive in b / 8: x[t] comes
// from HBM into that XCD's L2 once and is re-read from there for its other
// destinations.  Every thread issues one 16-byte load and kDestGroup 16-byte
// nontemporal stores.  Many short workgroups with few stores each write HBM
// faster than long-lived groups that each store a row many times: rows-only
// dispatch at 4096 tokens, H = 7168, R = 64, x cold, 95 against 104 us in
// the whole step (896 threads, two destinations per workgroup; one
// destination exposed the row load's latency once per store: 135 us).
//
// With top-k outputs the first ntk workgroups (a multiple of 8, so the row
// workgroups keep their XCDs) write them row-major: BT / K consecutive
// destination rows each, lane (row, k) -- the row's source token from
// recv_src_idx, its rank by a binary search of the rank segment ends
// (rank_prefix_matrix, whose last entry is N).  Every line of the top-k
// outputs is then written by one workgroup; written by the row workgroups
// instead (one 64- and one 32-byte piece per row and workgroup) they cost
// 13 us at the training-scale batch.
constexpr int kDestGroup = 2;

template <int BT, bool kTopk>
__global__ __launch_bounds__(BT) void dispatch_scatter_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int epr, int kmax, int ny,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    u32x4 *__restrict__ recv_x, int64_t *__restrict__ recv_topk_idx,
    float *__restrict__ recv_topk_weights, const int32_t *__restrict__ recv_src_idx,
    const int32_t *__restrict__ rank_prefix, int R, int ntk)
{
    unsigned b = blockIdx.x;
    if (kTopk) {
        if (b < unsigned(ntk)) {
            __shared__ int32_t s_end[kMaxRanks];
            const int tid = threadIdx.x;
            for (int r = tid; r < R; r += BT)
                s_end[r] = rank_prefix[r];
            __syncthreads();
            const int q = BT / K;  // rows of this workgroup
            const int jr = tid / K;
            const int k = tid - jr * K;
            const int64_t j = int64_t(b) * q + jr;
            if (jr >= q || j >= s_end[R - 1])
                return;
            int lo = 0, hi = R - 1;  // rank of row j: the first segment ending past it
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_end[mid] > j)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int64_t t = recv_src_idx[j];
            const int64_t e = topk_idx[t * K + k];
            const bool mine = e >= 0 && e < E && int(e) / epr == lo;
            if (recv_topk_idx != nullptr)
                recv_topk_idx[j * K + k] = mine ? e - int64_t(lo) * epr : -1;
            if (recv_topk_weights != nullptr)
                recv_topk_weights[j * K + k] = mine ? topk_weights[t * K + k] : 0.0f;
            return;
        }
        b -= unsigned(ntk);
    }
    const unsigned groups = unsigned((kmax + kDestGroup - 1) / kDestGroup);
    const unsigned per_tok = groups * unsigned(ny);
    const unsigned i = b >> 3;
    const unsigned u = i / per_tok;
    const int t = int(u * 8 + (b & 7));
    if (t >= T)
        return;
    const unsigned rem = i - u * per_tok;
    const int g = int(rem / unsigned(ny));
    const int yb = int(rem - unsigned(g) * unsigned(ny));
    const int c = yb * BT + int(threadIdx.x);
    // the row's load does not depend on the destinations: issued first
    u32x4 v = {0, 0, 0, 0};
    if (recv_x != nullptr)
        v = x[int64_t(t) * V + (c < V ? c : V - 1)];
    if (recv_x == nullptr || c >= V)
        return;
    for (int j = 0; j < kDestGroup; ++j) {
        const int k = g * kDestGroup + j;
        if (k >= kmax)
            break;
        const int row = dst_row[int64_t(t) * kmax + k];  // rows are packed first, then -1
        if (row < 0)
            break;
        __builtin_nontemporal_store(v, recv_x + int64_t(row) * V + c);
    }
}

// The two kernels share one argument list; the scatter kernel takes its
// chunk count ny where the token-major kernel takes S.
typedef void (*PackFn)(const u32x4 *, int, int, int, int, int, int, int, const int32_t *,
                       const int32_t *, const int64_t *, const float *, u32x4 *, int64_t *,
                       float *, const int32_t *, const int32_t *, int, int);

// A launch shape.  Token-major: G lanes per group, VPT vectors per lane, S
// groups per token (row slices), NTS / NTL nontemporal stores / loads, P
// persistent block count (0: one group per token slice).  Scatter
// (destination-major): G threads per workgroup, one vector each.  The tuning
// knob addresses shapes as (G, VPT, scatter*10000 + S*1000 + NTL*100 +
// NTS*10 + P/256).
struct PackCfg {
    int G, VPT, S, NTS, NTL, P;
    PackFn plain, topk;
    int scatter;
};

#define EP_PACK_CFG(G, VPT, S, NTS, NTL, P)                                                \
    {G, VPT, S, NTS, NTL, P, dispatch_pack_kernel<G, VPT, NTS, NTL, false>,                \
     dispatch_pack_kernel<G, VPT, NTS, NTL, true>, 0}
#define EP_SCATTER_CFG(BT)                                                                  \
    {BT, 1, 1, 1, 0, 0, dispatch_scatter_kernel<BT, false>, dispatch_scatter_kernel<BT, true>, 1}

const PackCfg kPackCfgs[] = {
    EP_SCATTER_CFG(128), EP_SCATTER_CFG(448), EP_SCATTER_CFG(896), EP_SCATTER_CFG(640),
    EP_SCATTER_CFG(768),
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
    return c.scatter * 10000 + c.S * 1000 + c.NTL * 100 + c.NTS * 10 + c.P / 256;
}

// Top-k writer workgroups of the scatter kernel: BT / K rows each for the
// T * kmax rows there can be, rounded up to a multiple of 8.
int64_t scatter_topk_blocks(const LayoutShape &s, int bt)
{
    const int64_t q = bt / s.K;
    const int64_t n = (int64_t(s.T) * s.kmax + q - 1) / q;
    return (n + 7) / 8 * 8;
}

// Workgroups of the scatter kernel's rows for this shape, or 0 when the
// grid (with its top-k writers) would not fit (the token-major kernel then
// takes the launch).
int64_t scatter_blocks(const LayoutShape &s, int V, int bt)
{
    const int64_t ny = (V + bt - 1) / bt;
    const int64_t b = int64_t((s.T + 7) / 8) * 8 * ((s.kmax + kDestGroup - 1) / kDestGroup) * ny;
    return b + scatter_topk_blocks(s, bt) < (int64_t(1) << 31) ? b : 0;
}

std::atomic<int> g_over_g{-2}, g_over_v{-1}, g_over_c{-1};  // -2: env not read yet

// Launch shape for a row of V vectors.  An override (ep_set_tuning, or the
// env var EP_TUNE_DISPATCH="G,VPT,code") wins; results never depend on it.
// Otherwise the scatter kernel with 896 threads per workgroup when they cut
// the row into whole chunks (H = 7168: one chunk per row; 96 against 99 us
// for 448 threads in the training-scale step, 102-121 us for 256, 512 or
// 640), else with 448; a grid too large for it takes the token-major kernel,
// with one chunk that covers the row exactly, the most lanes, nontemporal
// stores and one group per token.
const PackCfg &pick_token_major(int V)
{
    for (int G : {128, 256, 64})
        for (const PackCfg &c : kPackCfgs)
            if (!c.scatter && c.G == G && c.G * c.VPT == V && c.S == 1 && c.NTS == 1 &&
                c.NTL == 0 && c.P == 0)
                return c;
    const int vpt = V <= 256 ? 1 : V <= 512 ? 2 : 4;  // 256 lanes x 1, 2 or 4 (all compiled in)
    for (const PackCfg &c : kPackCfgs)
        if (!c.scatter && c.G == 256 && c.VPT == vpt && c.S == 1 && c.P == 0)
            return c;
    __builtin_unreachable();
}

// The compiled-in scatter shape with bt threads (448 and 896 are).
const PackCfg &scatter_cfg(int bt)
{
    for (const PackCfg &c : kPackCfgs)
        if (c.scatter && c.G == bt)
            return c;
    __builtin_unreachable();
}

const PackCfg &pick(const LayoutShape &s, int V)
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
            return c.scatter && scatter_blocks(s, V, c.G) == 0 ? pick_token_major(V) : c;
    const PackCfg &sc = scatter_cfg(V % 896 == 0 ? 896 : 448);
    if (scatter_blocks(s, V, sc.G) > 0)
        return sc;
    return pick_token_major(V);
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
    const bool topk = recv_topk_idx != nullptr || recv_topk_weights != nullptr;
    const PackCfg &c = pick(s, V);
    if (c.scatter) {
        const int ny = (V + c.G - 1) / c.G;
        // top-k writers: BT / K rows each, for the T * kmax rows there can be
        const int64_t ntk = topk ? scatter_topk_blocks(s, c.G) : 0;
        const int64_t blocks = scatter_blocks(s, V, c.G) + ntk;
        if (log_enabled())
            log_launch("dispatch_scatter T=%d H=%d K=%d R=%d: BT=%d chunks=%d blocks=%lld%s",
                       s.T, hidden, s.K, s.R, c.G, ny, (long long)blocks, topk ? " +topk" : "");
        hipLaunchKernelGGL(topk ? c.topk : c.plain, dim3(unsigned(blocks)), dim3(c.G), 0, stream,
                           static_cast<const u32x4 *>(x), s.T, V, s.K, s.E, s.epr, s.kmax, ny,
                           b.dst_row, b.dst_rank, topk_idx, topk_weights,
                           static_cast<u32x4 *>(recv_x), recv_topk_idx, recv_topk_weights,
                           b.recv_src_idx, b.rank_prefix_matrix, s.R, int(ntk));
        return hipGetLastError();
    }
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
                       recv_topk_idx, recv_topk_weights, nullptr, nullptr, 0, 0);
    return hipGetLastError();
}

}  // namespace ep

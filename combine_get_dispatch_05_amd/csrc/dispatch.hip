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
// Token-major: one workgroup per token reads the row from HBM once into
// VGPRs (16-byte vectors, fully coalesced) and stores it to each of the
// token's destination rows (at most min(K, R), from the layout's per-token
// row list).  Reading x once and streaming the copies keeps the kernel at the
// algorithmic byte count whatever the segment sizes; skewed routing only
// changes how many stores a workgroup issues.  Stores are nontemporal: the
// packed rows are not re-read by this kernel, so they should not evict the
// rows still to be read from the L2/MALL.

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kPackBlock = 256;

template <int VPT, bool kTopk>
__global__ __launch_bounds__(kPackBlock) void dispatch_pack_kernel(
    const u32x4 *__restrict__ x, int V, int K, int E, int epr, int kmax,
    const int32_t *__restrict__ dst_row, const int32_t *__restrict__ dst_rank,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    u32x4 *__restrict__ recv_x, int64_t *__restrict__ recv_topk_idx,
    float *__restrict__ recv_topk_weights)
{
    __shared__ int32_t s_row[kMaxTopk];
    __shared__ int32_t s_rank[kMaxTopk];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    if (tid < kmax) {
        s_row[tid] = dst_row[t * kmax + tid];
        s_rank[tid] = dst_rank[t * kmax + tid];
    }
    __syncthreads();
    int nhit = 0;
    while (nhit < kmax && s_row[nhit] >= 0)
        ++nhit;

    if (recv_x != nullptr) {
        const u32x4 *src = x + t * V;
        for (int base = 0; base < V; base += kPackBlock * VPT) {
            u32x4 v[VPT];
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kPackBlock + tid;
                if (idx < V)
                    v[i] = src[idx];
            }
            for (int j = 0; j < nhit; ++j) {
                u32x4 *dst = recv_x + int64_t(s_row[j]) * V;
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int idx = base + i * kPackBlock + tid;
                    if (idx < V)
                        __builtin_nontemporal_store(v[i], dst + idx);
                }
            }
        }
    }

    if (kTopk) {
        for (int p = tid; p < nhit * K; p += kPackBlock) {
            const int j = p / K;
            const int k = p - j * K;
            const int64_t row = s_row[j];
            const int r = s_rank[j];
            const int64_t e = topk_idx[t * K + k];
            const bool mine = e >= 0 && e < E && int(e) / epr == r;
            if (recv_topk_idx != nullptr)
                recv_topk_idx[row * K + k] = mine ? e - int64_t(r) * epr : -1;
            if (recv_topk_weights != nullptr)
                recv_topk_weights[row * K + k] = mine ? topk_weights[t * K + k] : 0.0f;
        }
    }
}

template <int VPT>
hipError_t launch_vpt(const LayoutShape &s, int V, const void *x, const LayoutBufs &b,
                      const int64_t *topk_idx, const float *topk_weights, void *recv_x,
                      int64_t *recv_topk_idx, float *recv_topk_weights, hipStream_t stream)
{
    const bool topk = recv_topk_idx != nullptr || recv_topk_weights != nullptr;
    if (topk)
        hipLaunchKernelGGL((dispatch_pack_kernel<VPT, true>), dim3(s.T), dim3(kPackBlock), 0,
                           stream, static_cast<const u32x4 *>(x), V, s.K, s.E, s.epr, s.kmax,
                           b.dst_row, b.dst_rank, topk_idx, topk_weights,
                           static_cast<u32x4 *>(recv_x), recv_topk_idx, recv_topk_weights);
    else
        hipLaunchKernelGGL((dispatch_pack_kernel<VPT, false>), dim3(s.T), dim3(kPackBlock), 0,
                           stream, static_cast<const u32x4 *>(x), V, s.K, s.E, s.epr, s.kmax,
                           b.dst_row, b.dst_rank, topk_idx, topk_weights,
                           static_cast<u32x4 *>(recv_x), recv_topk_idx, recv_topk_weights);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const LayoutShape &s, int hidden, const void *x, const LayoutBufs &b,
                           const int64_t *topk_idx, const float *topk_weights, void *recv_x,
                           int64_t *recv_topk_idx, float *recv_topk_weights, hipStream_t stream)
{
    if (s.T == 0)
        return hipSuccess;
    const int V = hidden / 8;
    const int need = (V + kPackBlock - 1) / kPackBlock;
    if (need <= 1)
        return launch_vpt<1>(s, V, x, b, topk_idx, topk_weights, recv_x, recv_topk_idx,
                             recv_topk_weights, stream);
    if (need <= 2)
        return launch_vpt<2>(s, V, x, b, topk_idx, topk_weights, recv_x, recv_topk_idx,
                             recv_topk_weights, stream);
    return launch_vpt<4>(s, V, x, b, topk_idx, topk_weights, recv_x, recv_topk_idx,
                         recv_topk_weights, stream);
}

}  // namespace ep

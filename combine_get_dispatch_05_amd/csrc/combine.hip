// combine.hip -- combine gather-reduce on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "Combine Operation": the rows a token sent out come back and are reduced by
// addition into that token's position, using the dispatch handle to find
// them.  Here the rows of token t sit at S[r] + send_head[t][r] in one buffer;
// the workgroup for t reads them in ascending rank order (the layout's
// per-token row list is already in that order), adds them in fp32 registers
// starting from +0, and writes one bf16 row rounded to nearest even.  The
// optional weight reduction sums the per-row top-k weights the same way.
//
// The sum order is fixed (rank ascending, one add per row per element), so the
// result does not depend on launch geometry.  Two rows' loads are issued
// before either is added so that each lane keeps 2*VPT 16-byte loads in
// flight.

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kCombineBlock = 256;

template <int VPT>
__device__ __forceinline__ void add_rows(float (&acc)[VPT][8], const u32x4 (&v)[VPT])
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

template <int VPT>
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(
    const u32x4 *__restrict__ y, int V, int K, int kmax, const int32_t *__restrict__ dst_row,
    const float *__restrict__ recv_topk_weights, u32x4 *__restrict__ out,
    float *__restrict__ combined_topk_weights)
{
    __shared__ int32_t s_row[kMaxTopk];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    if (tid < kmax)
        s_row[tid] = dst_row[t * kmax + tid];
    __syncthreads();
    int nhit = 0;
    while (nhit < kmax && s_row[nhit] >= 0)
        ++nhit;

    for (int base = 0; base < V; base += kCombineBlock * VPT) {
        float acc[VPT][8];
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;

        int j = 0;
        for (; j + 1 < nhit; j += 2) {
            const u32x4 *ya = y + int64_t(s_row[j]) * V;
            const u32x4 *yb = y + int64_t(s_row[j + 1]) * V;
            u32x4 a[VPT], c[VPT];
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kCombineBlock + tid;
                a[i] = idx < V ? ya[idx] : u32x4{0, 0, 0, 0};
                c[i] = idx < V ? yb[idx] : u32x4{0, 0, 0, 0};
            }
            add_rows<VPT>(acc, a);
            add_rows<VPT>(acc, c);
        }
        if (j < nhit) {
            const u32x4 *ya = y + int64_t(s_row[j]) * V;
            u32x4 a[VPT];
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kCombineBlock + tid;
                a[i] = idx < V ? ya[idx] : u32x4{0, 0, 0, 0};
            }
            add_rows<VPT>(acc, a);
        }

        u32x4 *o = out + t * V;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = base + i * kCombineBlock + tid;
            if (idx < V) {
                u32x4 r;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
                __builtin_nontemporal_store(r, o + idx);
            }
        }
    }

    if (combined_topk_weights != nullptr) {
        for (int k = tid; k < K; k += kCombineBlock) {
            float w = 0.0f;
            for (int jj = 0; jj < nhit; ++jj)
                w += recv_topk_weights[int64_t(s_row[jj]) * K + k];
            combined_topk_weights[t * K + k] = w;
        }
    }
}

template <int VPT>
hipError_t launch_vpt(const LayoutShape &s, int V, const void *y, const LayoutBufs &b,
                      const float *recv_topk_weights, void *out, float *combined_topk_weights,
                      hipStream_t stream)
{
    hipLaunchKernelGGL((combine_kernel<VPT>), dim3(s.T), dim3(kCombineBlock), 0, stream,
                       static_cast<const u32x4 *>(y), V, s.K, s.kmax, b.dst_row,
                       recv_topk_weights, static_cast<u32x4 *>(out), combined_topk_weights);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const LayoutShape &s, int hidden, const void *y, const LayoutBufs &b,
                          const float *recv_topk_weights, void *out,
                          float *combined_topk_weights, hipStream_t stream)
{
    if (s.T == 0)
        return hipSuccess;
    const int V = hidden / 8;
    const int need = (V + kCombineBlock - 1) / kCombineBlock;
    if (need <= 1)
        return launch_vpt<1>(s, V, y, b, recv_topk_weights, out, combined_topk_weights, stream);
    if (need <= 2)
        return launch_vpt<2>(s, V, y, b, recv_topk_weights, out, combined_topk_weights, stream);
    return launch_vpt<4>(s, V, y, b, recv_topk_weights, out, combined_topk_weights, stream);
}

}  // namespace ep

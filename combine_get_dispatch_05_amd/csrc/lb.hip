// lb.hip -- load-balance operations over redundant expert replicas, and the
// rank-mask utility.
//
// "Chapter 10, V2: buffers beyond EP", section 10.2: lb_prefetch_weights
// copies each expert's weights into the slots of its redundant replicas
// before the expert computation; lb_reduce_grads folds the replicas'
// gradients back into the experts they copy during the backward pass; both
// follow a redundancy mapping (replica j copies expert mapping[j]).
// Readings: bf16 tensors [experts][elems] and [replicas][elems]; the
// reduction accumulates in fp32 starting from the expert's own gradient,
// adds its replicas in ascending replica order and rounds once; mapping
// entries outside [0, E) are ignored.
//
// Both are streaming copies/reductions bound by HBM bandwidth: one workgroup
// per (replica, 2048-element chunk), 16-byte vectors, two vectors per lane.
// In the reduction only the workgroup of an expert's first replica works (it
// walks all of that expert's replicas in order, finding them with wave-wide
// ballots over the mapping), so every output element is written once, in a
// fixed order, with no atomics.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "Dynamic Rank Masking": low_latency_update_mask_buffer / clean_mask_buffer
// set entries of a per-rank mask (0 active, 1 masked) that the low-latency
// kernels read.  They are written by a one-block kernel (no memset), so the
// calls are stream-ordered like every other call.

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLBBlock = 256;
constexpr int kLBVec = 2;  // 16-byte vectors per lane
constexpr int64_t kLBChunk = int64_t(kLBBlock) * kLBVec * 8;  // bf16 elements per workgroup

__global__ __launch_bounds__(kLBBlock) void lb_reduce_grads_kernel(
    const u32x4 *__restrict__ redundant, u32x4 *__restrict__ expert,
    const int64_t *__restrict__ mapping, int num_replicas, int num_experts, int64_t vecs)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int j = blockIdx.y;
    const int64_t e = mapping[j];
    if (e < 0 || e >= num_experts)
        return;
    // An earlier replica of e does the work.  The mapping is scanned 64
    // entries per wave-wide load; every wave of the block reaches the same
    // answer, and the kernel has no barrier.
    for (int c = 0; c < j; c += kWave) {
        const int jj = c + lane;
        if (wave_ballot(jj < j && mapping[jj] == e) != 0)
            return;
    }
    const int64_t v0 = int64_t(blockIdx.x) * kLBBlock * kLBVec;
    float acc[kLBVec][8];
    u32x4 cur[kLBVec];
#pragma unroll
    for (int i = 0; i < kLBVec; ++i) {
        const int64_t idx = v0 + i * kLBBlock + threadIdx.x;
        cur[i] = idx < vecs ? expert[e * vecs + idx] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[i][2 * q] = bf16_lo(cur[i][q]);
            acc[i][2 * q + 1] = bf16_hi(cur[i][q]);
        }
    }
    // e's replicas from j on, in ascending order: a ballot per 64 entries,
    // then its set bits lowest first.
    for (int c = j; c < num_replicas; c += kWave) {
        const int jc = c + lane;
        uint64_t hits = wave_ballot(jc < num_replicas && mapping[jc] == e);
        while (hits) {
            const int64_t jj = c + __ffsll((unsigned long long)hits) - 1;
            hits &= hits - 1;
#pragma unroll
            for (int i = 0; i < kLBVec; ++i) {
                const int64_t idx = v0 + i * kLBBlock + threadIdx.x;
                const u32x4 rv = idx < vecs
                                     ? __builtin_nontemporal_load(redundant + jj * vecs + idx)
                                     : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[i][2 * q] += bf16_lo(rv[q]);
                    acc[i][2 * q + 1] += bf16_hi(rv[q]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kLBVec; ++i) {
        const int64_t idx = v0 + i * kLBBlock + threadIdx.x;
        if (idx < vecs) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
            expert[e * vecs + idx] = o;
        }
    }
}

__global__ __launch_bounds__(kLBBlock) void lb_prefetch_weights_kernel(
    const u32x4 *__restrict__ expert, u32x4 *__restrict__ redundant,
    const int64_t *__restrict__ mapping, int num_experts, int64_t vecs)
{
    const int j = blockIdx.y;
    const int64_t e = mapping[j];
    if (e < 0 || e >= num_experts)
        return;
    const int64_t v0 = int64_t(blockIdx.x) * kLBBlock * kLBVec;
    u32x4 v[kLBVec];
#pragma unroll
    for (int i = 0; i < kLBVec; ++i) {
        const int64_t idx = v0 + i * kLBBlock + threadIdx.x;
        if (idx < vecs)
            v[i] = __builtin_nontemporal_load(expert + e * vecs + idx);
    }
#pragma unroll
    for (int i = 0; i < kLBVec; ++i) {
        const int64_t idx = v0 + i * kLBBlock + threadIdx.x;
        if (idx < vecs)
            __builtin_nontemporal_store(v[i], redundant + int64_t(j) * vecs + idx);
    }
}

__global__ void mask_set_kernel(int32_t *mask, int num_ranks, int rank, int value)
{
    for (int r = threadIdx.x; r < num_ranks; r += blockDim.x)
        if (rank < 0 || r == rank)
            mask[r] = value;
}

}  // namespace

hipError_t launch_lb_reduce_grads(const void *redundant_grads, void *expert_grads,
                                  const int64_t *mapping, int num_replicas, int num_experts,
                                  int64_t elems, hipStream_t stream)
{
    if (num_replicas == 0 || elems == 0)
        return hipSuccess;
    const int64_t vecs = elems / 8;
    const int64_t chunks = (elems + kLBChunk - 1) / kLBChunk;
    hipLaunchKernelGGL(lb_reduce_grads_kernel, dim3(unsigned(chunks), num_replicas),
                       dim3(kLBBlock), 0, stream, static_cast<const u32x4 *>(redundant_grads),
                       static_cast<u32x4 *>(expert_grads), mapping, num_replicas, num_experts,
                       vecs);
    return hipGetLastError();
}

hipError_t launch_lb_prefetch_weights(const void *expert_weights, void *redundant_weights,
                                      const int64_t *mapping, int num_replicas, int num_experts,
                                      int64_t elems, hipStream_t stream)
{
    if (num_replicas == 0 || elems == 0)
        return hipSuccess;
    const int64_t vecs = elems / 8;
    const int64_t chunks = (elems + kLBChunk - 1) / kLBChunk;
    hipLaunchKernelGGL(lb_prefetch_weights_kernel, dim3(unsigned(chunks), num_replicas),
                       dim3(kLBBlock), 0, stream, static_cast<const u32x4 *>(expert_weights),
                       static_cast<u32x4 *>(redundant_weights), mapping, num_experts, vecs);
    return hipGetLastError();
}

hipError_t launch_mask_set(int32_t *mask, int num_ranks, int rank, int value, hipStream_t stream)
{
    hipLaunchKernelGGL(mask_set_kernel, dim3(1), dim3(256), 0, stream, mask, num_ranks, rank,
                       value);
    return hipGetLastError();
}

}  // namespace ep

// check.hip -- debug check of the handle-reuse contract.
//
// "How DeepEP Optimizes Handle Reuse for Repeated Dispatches" ("Performance
// Contract and Constraints"): a handle's layout is only valid for the top-k
// table it was computed from; reusing it after the routing changed is
// undefined.  With EP_CHECK=1 in the environment the library stores a 64-bit
// hash of that table in the handle and compares it with the hash of the
// table a later dispatch passes along with the handle.
//
// The hash is a sum over the entries of SplitMix64's finalizer applied to
// (index * golden-ratio constant) xor value: a sum, so the order in which
// lanes and workgroups add their parts does not change it.

#include "ep_internal.h"

namespace ep {

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z ^= z >> 30;
    z *= 0xbf58476d1ce4e5b9ull;
    z ^= z >> 27;
    z *= 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

__global__ void hash_zero_kernel(unsigned long long *out) { *out = 0; }

__global__ __launch_bounds__(256) void topk_hash_kernel(const int64_t *__restrict__ topk,
                                                        int64_t n,
                                                        unsigned long long *__restrict__ out)
{
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    uint64_t acc = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        acc += mix64((uint64_t(i) * 0x9e3779b97f4a7c15ull) ^ uint64_t(topk[i]));
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        acc += __shfl_xor((unsigned long long)acc, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0)
        atomicAdd(out, (unsigned long long)acc);
}

}  // namespace

hipError_t launch_topk_hash(const int64_t *topk_idx, int64_t n, uint64_t *out, hipStream_t stream)
{
    unsigned long long *o = reinterpret_cast<unsigned long long *>(out);
    hipLaunchKernelGGL(hash_zero_kernel, dim3(1), dim3(1), 0, stream, o);
    if (n > 0) {
        int64_t blocks = (n + 255) / 256;
        blocks = blocks > 1024 ? 1024 : blocks;
        hipLaunchKernelGGL(topk_hash_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           topk_idx, n, o);
    }
    return hipGetLastError();
}

}  // namespace ep

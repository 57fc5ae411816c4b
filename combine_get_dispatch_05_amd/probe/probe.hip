// probe.hip -- measurement kernels of libep_probe.so (declared in
// include/ep_probe.h): plain streaming kernels that move the same bytes as
// the library's operations, as ceilings for the benchmark.  They compute
// nothing of the method and share no code with libep.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_probe.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kG = 128;  // lanes per token (as the pack and the combine)
constexpr int kVPT = 7;  // 16-byte vectors per lane per pass (H = 7168: one pass)

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t rne16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void write_kernel(v4u *__restrict__ dst, int64_t n)
{
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
        const v4u v = {uint32_t(i), uint32_t(i >> 32), 0x3f803f80u, 0x40004000u};
        __builtin_nontemporal_store(v, dst + i);
    }
}

// One pass over [base, base + kG*kVPT) of a token's row: every load issued
// (index clamped into the row) before the plane count is looked at, then
// the chunk stored to n planes.
__device__ __forceinline__ void pack_chunk(const v4u *__restrict__ src, v4u *__restrict__ planes,
                                           int T, int V, int t, int base, int g, int r, int kmax)
{
    v4u v[kVPT];
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
        const int c = base + i * kG + g;
        v[i] = src[c < V ? c : V - 1];
    }
#pragma unroll
    for (int i = 0; i < kVPT; ++i)
        asm volatile("" : "+v"(v[i]));  // keep the loads here, ahead of the count
    asm volatile("" : "+v"(r));          // and the count's use behind them
    const int n = r < 0 ? 0 : (r > kmax ? kmax : r);
    for (int j = 0; j < n; ++j) {
        v4u *dst = planes + (int64_t(j) * T + t) * V;
#pragma unroll
        for (int i = 0; i < kVPT; ++i) {
            const int c = base + i * kG + g;
            if (c < V)
                __builtin_nontemporal_store(v[i], dst + c);
        }
    }
}

__global__ __launch_bounds__(256) void pack_kernel(const v4u *__restrict__ x, int T, int V,
                                                   const int32_t *__restrict__ rows, int kmax,
                                                   v4u *__restrict__ planes)
{
    const int t = blockIdx.x * (256 / kG) + threadIdx.x / kG;
    const int g = threadIdx.x % kG;
    if (t >= T)
        return;
    const int r = rows[t];
    const v4u *src = x + int64_t(t) * V;
    if (V <= kG * kVPT)
        pack_chunk(src, planes, T, V, t, 0, g, r, kmax);
    else
        for (int base = 0; base < V; base += kG * kVPT)
            pack_chunk(src, planes, T, V, t, base, g, r, kmax);
}

__global__ __launch_bounds__(256) void reduce_kernel(const v4u *__restrict__ planes, int T, int V,
                                                     const int32_t *__restrict__ rows, int kmax,
                                                     v4u *__restrict__ out)
{
    const int t = blockIdx.x * (256 / kG) + threadIdx.x / kG;
    const int g = threadIdx.x % kG;
    if (t >= T)
        return;
    const int n = rows[t] < 0 ? 0 : (rows[t] > kmax ? kmax : rows[t]);
    for (int base = 0; base < V; base += kG * kVPT) {
        float acc[kVPT][8];
#pragma unroll
        for (int i = 0; i < kVPT; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;
        for (int j = 0; j < n; ++j) {
            const v4u *src = planes + (int64_t(j) * T + t) * V;
            v4u v[kVPT];
#pragma unroll
            for (int i = 0; i < kVPT; ++i) {
                const int c = base + i * kG + g;
                v[i] = c < V ? __builtin_nontemporal_load(src + c) : v4u{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < kVPT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[i][2 * q] += lo16(v[i][q]);
                    acc[i][2 * q + 1] += hi16(v[i][q]);
                }
        }
#pragma unroll
        for (int i = 0; i < kVPT; ++i) {
            const int c = base + i * kG + g;
            if (c < V) {
                v4u r;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    r[q] = rne16(acc[i][2 * q]) | (rne16(acc[i][2 * q + 1]) << 16);
                __builtin_nontemporal_store(r, out + int64_t(t) * V + c);
            }
        }
    }
}

__global__ void empty_kernel(int *flag)
{
    if (flag != nullptr && threadIdx.x == 0 && blockIdx.x == 0x7fffffff)
        *flag = 1;
}

constexpr int kLLCopyBlock = 512;

__global__ __launch_bounds__(kLLCopyBlock) void ll_copy_kernel(const v4u *__restrict__ x, int V,
                                                               int K, int ny,
                                                               v4u *__restrict__ cells)
{
    const int t = blockIdx.x / ny;
    const int yb = blockIdx.x - t * ny;
    const int per = (V + ny - 1) / ny;
    const int c0 = yb * per;
    const int c1 = c0 + per < V ? c0 + per : V;
    for (int c = c0 + threadIdx.x; c < c1; c += kLLCopyBlock) {
        const v4u v = x[int64_t(t) * V + c];
        for (int k = 0; k < K; ++k)
            cells[(int64_t(t) * K + k) * V + c] = v;
    }
}

__global__ __launch_bounds__(256) void ll_reduce_kernel(const v4u *__restrict__ cells,
                                                        const float *__restrict__ w, int V, int K,
                                                        v4u *__restrict__ out)
{
    const int64_t t = blockIdx.x;
    const int idx = blockIdx.y * 256 + threadIdx.x;
    if (idx >= V)
        return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k0 = 0; k0 < K; k0 += 8) {
        v4u v[8];
#pragma unroll
        for (int g = 0; g < 8; ++g)
            v[g] = k0 + g < K ? cells[(t * K + k0 + g) * V + idx] : v4u{0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (k0 + g < K) {
                const float wk = w[t * K + k0 + g];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = __builtin_fmaf(wk, lo16(v[g][q]), acc[2 * q]);
                    acc[2 * q + 1] = __builtin_fmaf(wk, hi16(v[g][q]), acc[2 * q + 1]);
                }
            }
        }
    }
    v4u r;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r[q] = rne16(acc[2 * q]) | (rne16(acc[2 * q + 1]) << 16);
    out[t * V + idx] = r;
}

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

}  // namespace

extern "C" {

int ep_probe_write(void *dst, int64_t bytes, ep_stream_t stream)
{
    if (dst == nullptr || bytes < 0)
        return EP_ERR_INVALID;
    if (bytes % 16 != 0 || !al16(dst))
        return EP_ERR_ALIGN;
    const int64_t n = bytes / 16;
    if (n == 0)
        return EP_OK;
    int64_t blocks = (n + 4 * 256 - 1) / (4 * 256);
    blocks = blocks > 65536 ? 65536 : blocks;
    hipLaunchKernelGGL(write_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<v4u *>(dst), n);
    return status(hipGetLastError());
}

int ep_probe_pack(const void *x, int32_t T, int32_t hidden, const int32_t *rows_per_token,
                  int32_t kmax, void *planes, ep_stream_t stream)
{
    if (T < 0 || hidden <= 0 || kmax < 0 || (T > 0 && (x == nullptr || planes == nullptr ||
                                                        rows_per_token == nullptr)))
        return EP_ERR_INVALID;
    if (hidden % 8 != 0 || !al16(x) || !al16(planes))
        return EP_ERR_ALIGN;
    if (T == 0)
        return EP_OK;
    hipLaunchKernelGGL(pack_kernel, dim3(unsigned((T + 1) / 2)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u *>(x), T,
                       hidden / 8, rows_per_token, kmax, static_cast<v4u *>(planes));
    return status(hipGetLastError());
}

int ep_probe_reduce(const void *planes, int32_t T, int32_t hidden, const int32_t *rows_per_token,
                    int32_t kmax, void *out, ep_stream_t stream)
{
    if (T < 0 || hidden <= 0 || kmax < 0 || (T > 0 && (out == nullptr || planes == nullptr ||
                                                        rows_per_token == nullptr)))
        return EP_ERR_INVALID;
    if (hidden % 8 != 0 || !al16(out) || !al16(planes))
        return EP_ERR_ALIGN;
    if (T == 0)
        return EP_OK;
    hipLaunchKernelGGL(reduce_kernel, dim3(unsigned((T + 1) / 2)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u *>(planes), T,
                       hidden / 8, rows_per_token, kmax, static_cast<v4u *>(out));
    return status(hipGetLastError());
}

int ep_probe_empty(int32_t blocks, int32_t threads, ep_stream_t stream)
{
    if (blocks < 1 || threads < 64 || threads > 1024 || threads % 64 != 0)
        return EP_ERR_INVALID;
    hipLaunchKernelGGL(empty_kernel, dim3(unsigned(blocks)), dim3(unsigned(threads)), 0,
                       static_cast<hipStream_t>(stream), nullptr);
    return status(hipGetLastError());
}

int ep_probe_ll_copy(const void *x, int32_t T, int32_t hidden, int32_t K, void *cells,
                     ep_stream_t stream)
{
    if (T < 0 || hidden <= 0 || K < 1 || (T > 0 && (x == nullptr || cells == nullptr)))
        return EP_ERR_INVALID;
    if (hidden % 8 != 0 || !al16(x) || !al16(cells))
        return EP_ERR_ALIGN;
    if (T == 0)
        return EP_OK;
    const int V = hidden / 8;
    const int ny = (V + kLLCopyBlock - 1) / kLLCopyBlock;
    hipLaunchKernelGGL(ll_copy_kernel, dim3(unsigned(int64_t(T) * ny)), dim3(kLLCopyBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u *>(x), V, K, ny,
                       static_cast<v4u *>(cells));
    return status(hipGetLastError());
}

int ep_probe_ll_reduce(const void *cells, const float *w, int32_t T, int32_t hidden, int32_t K,
                       void *out, ep_stream_t stream)
{
    if (T < 0 || hidden <= 0 || K < 1 ||
        (T > 0 && (cells == nullptr || w == nullptr || out == nullptr)))
        return EP_ERR_INVALID;
    if (hidden % 8 != 0 || !al16(cells) || !al16(out))
        return EP_ERR_ALIGN;
    if (T == 0)
        return EP_OK;
    const int V = hidden / 8;
    hipLaunchKernelGGL(ll_reduce_kernel, dim3(unsigned(T), unsigned((V + 255) / 256)), dim3(256),
                       0, static_cast<hipStream_t>(stream), static_cast<const v4u *>(cells), w, V,
                       K, static_cast<v4u *>(out));
    return status(hipGetLastError());
}

}  // extern "C"

// ll.hip -- low-latency (decode) dispatch and combine on gfx950.
//
// "DeepEP Buffer Class API for Expert Parallel Communication", section
// "IB-GDA Kernels": low_latency_dispatch streams tokens straight into
// per-expert receive buffers with no intermediate staging and reports
// per-expert counts; low_latency_combine reduces the expert results back to
// the tokens' positions, weighted by the top-k weights.
//
// Dispatch is one fused launch with one workgroup per expert: the workgroup
// scans the [T][K] table, turns "names my expert" into slots with one
// block-wide prefix scan (so slots follow (token, slot) order), records the
// token of each slot, and then copies those token rows into the expert's
// area [le][r][slot][:] with every lane issuing independent 16-byte loads and
// stores.  No layout pass, no second launch, no host sync.
//
// Combine: one workgroup per (token, row chunk).  All K cell addresses of the
// token are resolved once into LDS; each lane then issues its K loads before
// the fused multiply-adds, which run in ascending slot order from +0.

#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kLLBlock = 256;
constexpr int kLLWaves = kLLBlock / kWave;

__device__ __forceinline__ int ll_wave_inclusive_scan(int v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(v, o, kWave);
        if (lane >= o)
            v += n;
    }
    return v;
}

// One workgroup per expert.  Each thread owns a contiguous chunk of the
// flattened [T][K] table (held in registers when it is short), counts the
// pairs naming its expert, and one block-wide exclusive scan of those counts
// gives every thread the first slot of its chunk, so slots follow (token,
// slot) order.  The rows are then copied with the (row, vector) pairs spread
// flat over the block, kUnroll independent 16-byte loads in flight per lane.
__global__ __launch_bounds__(kLLBlock) void ll_dispatch_kernel(
    const u32x4 *__restrict__ x, int T, int V, int K, int E, int R, int epr, int S,
    const int64_t *__restrict__ topk_idx, u32x4 *__restrict__ packed_x,
    int32_t *__restrict__ packed_count, int32_t *__restrict__ src_info,
    int32_t *__restrict__ topk_slot)
{
    constexpr int kHold = 8;
    __shared__ int32_t s_tok[kMaxLLSlots];
    __shared__ int32_t s_wsum[kLLWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int e = blockIdx.x;
    const int le = e % epr;
    const int r = e / epr;
    const int64_t cell0 = (int64_t(le) * R + r) * S;
    const int TK = T * K;
    const int chunk = (TK + kLLBlock - 1) / kLLBlock;
    const int i0 = tid * chunk;
    const int i1 = i0 + chunk < TK ? i0 + chunk : TK;
    const bool held = chunk <= kHold;

    int64_t v[kHold];
    int mine = 0;
    if (held) {
#pragma unroll
        for (int q = 0; q < kHold; ++q) {
            v[q] = i0 + q < i1 ? topk_idx[i0 + q] : -1;
            mine += v[q] == e ? 1 : 0;
        }
    } else {
        for (int i = i0; i < i1; ++i)
            mine += topk_idx[i] == e ? 1 : 0;
    }

    const int incl = ll_wave_inclusive_scan(mine);
    if (lane == kWave - 1)
        s_wsum[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kLLWaves; ++w) {
        const int c = s_wsum[w];
        before += w < wid ? c : 0;
        total += c;
    }
    int s = before + incl - mine;  // first slot of this thread's chunk

    auto place = [&](int i, int64_t val) {
        if (val == e) {
            if (s < S) {
                topk_slot[i] = s;
                src_info[cell0 + s] = i / K;
                s_tok[s] = i / K;
            } else {
                topk_slot[i] = -1;
            }
            ++s;
        } else if (e == 0 && !(val >= 0 && val < E)) {
            topk_slot[i] = -1;  // masked or invalid slots: workgroup 0 marks them
        }
    };
    if (held) {
#pragma unroll
        for (int q = 0; q < kHold; ++q)
            if (i0 + q < i1)
                place(i0 + q, v[q]);
    } else {
        for (int i = i0; i < i1; ++i)
            place(i, topk_idx[i]);
    }

    if (tid == 0)
        packed_count[int64_t(le) * R + r] = total;
    const int used = total < S ? total : S;
    for (int q = used + tid; q < S; q += kLLBlock)
        src_info[cell0 + q] = -1;
    __syncthreads();

    if (packed_x != nullptr) {
        constexpr int kUnroll = 8;
        const int n = used * V;
        for (int p0 = 0; p0 < n; p0 += kLLBlock * kUnroll) {
            u32x4 buf[kUnroll];
            int64_t dst[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int p = p0 + u * kLLBlock + tid;
                dst[u] = -1;
                if (p < n) {
                    const int row = p / V;
                    const int col = p - row * V;
                    buf[u] = x[int64_t(s_tok[row]) * V + col];
                    dst[u] = (cell0 + row) * V + col;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (dst[u] >= 0)
                    packed_x[dst[u]] = buf[u];
        }
    }
}

template <int VPT>
__global__ __launch_bounds__(kLLBlock) void ll_combine_kernel(
    const u32x4 *__restrict__ packed_y, int V, int K, int E, int R, int epr, int S,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    const int32_t *__restrict__ topk_slot, u32x4 *__restrict__ out)
{
    __shared__ int64_t s_cell[kMaxTopk];
    __shared__ float s_w[kMaxTopk];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    if (tid < K) {
        const int64_t e = topk_idx[t * K + tid];
        const int s = topk_slot[t * K + tid];
        const bool ok = e >= 0 && e < E && s >= 0 && s < S;
        s_cell[tid] = ok ? ((int64_t(int(e) % epr) * R + int(e) / epr) * S + s) : -1;
        s_w[tid] = topk_weights[t * K + tid];
    }
    __syncthreads();

    const int base = blockIdx.y * kLLBlock * VPT;
    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = 0.0f;

    constexpr int kGroup = 8;
    for (int k0 = 0; k0 < K; k0 += kGroup) {
        u32x4 v[kGroup][VPT];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            const int64_t cell = k < K ? s_cell[k] : -1;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = base + i * kLLBlock + tid;
                v[g][i] = (cell >= 0 && idx < V) ? packed_y[cell * V + idx] : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int k = k0 + g;
            if (k < K && s_cell[k] >= 0) {
                const float w = s_w[k];
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[i][2 * q] = __builtin_fmaf(w, bf16_lo(v[g][i][q]), acc[i][2 * q]);
                        acc[i][2 * q + 1] =
                            __builtin_fmaf(w, bf16_hi(v[g][i][q]), acc[i][2 * q + 1]);
                    }
                }
            }
        }
    }

    u32x4 *o = out + t * V;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int idx = base + i * kLLBlock + tid;
        if (idx < V) {
            u32x4 rv;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rv[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
            o[idx] = rv;
        }
    }
}

}  // namespace

hipError_t launch_ll_dispatch(const ep_dims &d, int num_slots, const void *x,
                              const int64_t *topk_idx, void *packed_x, int32_t *packed_count,
                              int32_t *src_info, int32_t *topk_slot, hipStream_t stream)
{
    const int E = d.num_experts, R = d.num_ranks;
    hipLaunchKernelGGL(ll_dispatch_kernel, dim3(E), dim3(kLLBlock), 0, stream,
                       static_cast<const u32x4 *>(x), d.num_tokens, d.hidden / 8, d.num_topk, E,
                       R, E / R, num_slots, topk_idx, static_cast<u32x4 *>(packed_x),
                       packed_count, src_info, topk_slot);
    return hipGetLastError();
}

hipError_t launch_ll_combine(const ep_dims &d, int num_slots, const void *packed_y,
                             const int64_t *topk_idx, const float *topk_weights,
                             const int32_t *topk_slot, void *out, hipStream_t stream)
{
    if (d.num_tokens == 0)
        return hipSuccess;
    const int E = d.num_experts, R = d.num_ranks;
    const int V = d.hidden / 8;
    constexpr int VPT = 1;
    const int chunks = (V + kLLBlock * VPT - 1) / (kLLBlock * VPT);
    hipLaunchKernelGGL((ll_combine_kernel<VPT>), dim3(d.num_tokens, chunks), dim3(kLLBlock), 0,
                       stream, static_cast<const u32x4 *>(packed_y), V, d.num_topk, E, R, E / R,
                       num_slots, topk_idx, topk_weights, topk_slot, static_cast<u32x4 *>(out));
    return hipGetLastError();
}

}  // namespace ep

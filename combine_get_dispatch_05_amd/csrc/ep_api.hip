// ep_api.hip -- host runtime and C ABI of libep.so (declared in include/ep.h).
//
// Owns argument validation ("Memory Alignment and Validation" of the DeepEP-Lib
// "Core Implementation" page: int4-multiple rows, aligned buffers), the
// dispatch handle ("What the Handle Contains" of "How DeepEP Optimizes Handle
// Reuse for Repeated Dispatches"), and a per-device pool of handle arenas,
// reused on the stream that freed them, so that creating a handle per step
// does not call hipMalloc after the first step.  Every kernel launch is enqueued on the caller's
// stream; the host only waits where the ABI says so (reading N back when a
// caller asks for it or when a buffer is smaller than the worst case).

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <dlfcn.h>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ep_internal.h"

using namespace ep;

namespace ep {

bool log_enabled()
{
    const char *v = std::getenv("EP_LOG");
    return v != nullptr && v[0] == '1';
}

void log_launch(const char *fmt, ...)
{
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(line, sizeof line, fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "[ep] %s\n", line);
}

}  // namespace ep

namespace {

thread_local std::string g_last_hip;

// EP_TRACE=1: a roctx range around every entry point, so rocprofv3's marker
// trace shows the calls over their kernels.  The roctx library is opened on
// first use only when the variable is set; without it nothing changes.
typedef int (*RangePushFn)(const char *);
typedef int (*RangePopFn)();

struct Roctx {
    RangePushFn push = nullptr;
    RangePopFn pop = nullptr;
};

const Roctx &roctx()
{
    static const Roctx r = [] {
        Roctx x;
        const char *v = std::getenv("EP_TRACE");
        if (v == nullptr || v[0] != '1')
            return x;
        void *h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
        if (h == nullptr)
            h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
        if (h == nullptr)
            return x;
        x.push = reinterpret_cast<RangePushFn>(dlsym(h, "roctxRangePushA"));
        x.pop = reinterpret_cast<RangePopFn>(dlsym(h, "roctxRangePop"));
        if (x.push == nullptr || x.pop == nullptr)
            x.push = nullptr, x.pop = nullptr;
        return x;
    }();
    return r;
}

struct TraceRange {
    bool on;
    explicit TraceRange(const char *name) : on(roctx().push != nullptr)
    {
        if (on)
            roctx().push(name);
    }
    ~TraceRange()
    {
        if (on)
            roctx().pop();
    }
};

int hip_fail(hipError_t e)
{
    g_last_hip = hipGetErrorString(e);
    return EP_ERR_HIP;
}

// ------------------------------------------------------------------ pool
//
// A freed arena remembers the stream it was freed on and is handed out again
// only to a later request on that same stream: stream order then puts the
// new user's work after every kernel that used the arena, so no event (and
// no event marker on the stream) is needed.  A request on another stream
// gets a fresh allocation, or an arena known to be idle.
//
// The pool is capped per device (kept bytes and arena count).  A free that
// takes it past the cap synchronizes the device once -- every arena freed
// before that point is then idle -- frees the oldest arenas until the pool
// is at half its byte cap and within its count, and marks the rest idle, so
// any stream may reuse them.  Only that path waits; the same-stream reuse
// path never does.  Trimming likewise synchronizes before it frees.

struct Arena {
    void *ptr = nullptr;
    size_t bytes = 0;
    hipStream_t freed_on = nullptr;
    bool idle = false;  // no work uses it any more: any stream may take it
    uint64_t seq = 0;   // order of freeing (oldest first out)
    LayoutCounters lc;  // the one-launch layout counters at the arena's start
};

struct DevicePool {
    std::mutex mu;
    std::vector<Arena> free_list;
    size_t kept = 0;  // bytes in free_list
    uint64_t seq = 0;
};

constexpr size_t kPoolMaxArenas = 64;

// Byte cap of each device's pool: EP_POOL_CAP_MB (read once), default 256 MiB.
size_t pool_cap_bytes()
{
    static const size_t cap = [] {
        const char *v = std::getenv("EP_POOL_CAP_MB");
        long long mb = v != nullptr ? std::atoll(v) : 256;
        if (mb < 1)
            mb = 1;
        return size_t(mb) << 20;
    }();
    return cap;
}

// Pools live until the process ends (never destroyed, so no HIP call runs
// from a static destructor after the runtime has gone).
DevicePool &pool_for(int dev)
{
    static std::mutex mu;
    static std::map<int, DevicePool *> pools;
    std::lock_guard<std::mutex> g(mu);
    DevicePool *&p = pools[dev];
    if (p == nullptr)
        p = new DevicePool();
    return *p;
}

size_t round_arena(size_t b)
{
    const size_t g = size_t(64) << 10;
    return b == 0 ? g : (b + g - 1) / g * g;
}

int trim_pool(DevicePool &P)
{
    std::vector<Arena> drop;
    {
        std::lock_guard<std::mutex> g(P.mu);
        drop.swap(P.free_list);
        P.kept = 0;
    }
    if (drop.empty())
        return EP_OK;
    int rc = EP_OK;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess)
        rc = hip_fail(e);
    for (auto &a : drop)
        (void)hipFree(a.ptr);
    return rc;
}

// Over the cap: one device-wide synchronization makes every arena freed
// before it idle; the oldest go back to HIP until the pool is at half its
// byte cap and within its arena count, and the others become reusable on any
// stream.  The current device is the pool's.
void shrink_pool(DevicePool &P)
{
    const size_t cap = pool_cap_bytes();
    uint64_t upto = 0;
    {
        std::lock_guard<std::mutex> g(P.mu);
        upto = P.seq;
    }
    if (hipDeviceSynchronize() != hipSuccess)
        return;  // leave the pool as it is; the error surfaces at the next call
    std::vector<Arena> drop;
    {
        std::lock_guard<std::mutex> g(P.mu);
        std::sort(P.free_list.begin(), P.free_list.end(),
                  [](const Arena &a, const Arena &b) { return a.seq < b.seq; });
        size_t i = 0;
        while (i < P.free_list.size() && P.free_list[i].seq <= upto &&
               (P.kept > cap / 2 || P.free_list.size() - i > kPoolMaxArenas / 2)) {
            P.kept -= P.free_list[i].bytes;
            drop.push_back(P.free_list[i]);
            ++i;
        }
        P.free_list.erase(P.free_list.begin(), P.free_list.begin() + i);
        for (Arena &a : P.free_list)
            if (a.seq <= upto)
                a.idle = true;
    }
    for (auto &a : drop)
        (void)hipFree(a.ptr);
}

int arena_get(int dev, size_t bytes, hipStream_t stream, Arena *out)
{
    bytes = round_arena(bytes);
    DevicePool &P = pool_for(dev);
    {
        std::lock_guard<std::mutex> g(P.mu);
        size_t best = P.free_list.size();
        for (size_t i = 0; i < P.free_list.size(); ++i) {
            const Arena &a = P.free_list[i];
            if (a.bytes < bytes || a.bytes > 2 * bytes || !(a.idle || a.freed_on == stream))
                continue;
            if (best == P.free_list.size() || a.bytes < P.free_list[best].bytes)
                best = i;
        }
        if (best < P.free_list.size()) {
            *out = P.free_list[best];
            P.kept -= out->bytes;
            P.free_list.erase(P.free_list.begin() + best);
            out->idle = false;
            return EP_OK;
        }
    }
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        trim_pool(P);
        e = hipMalloc(&p, bytes);
    }
    if (e == hipErrorOutOfMemory) {
        (void)hipGetLastError();
        return EP_ERR_NOMEM;
    }
    if (e != hipSuccess)
        return hip_fail(e);
    // the one-launch layout's counters start at zero in a new arena
    e = hipMemsetAsync(p, 0, kLayoutCtrBytes, stream);
    if (e != hipSuccess) {
        (void)hipFree(p);
        return hip_fail(e);
    }
    out->ptr = p;
    out->bytes = bytes;
    out->freed_on = stream;
    out->idle = false;
    out->lc = LayoutCounters();
    return EP_OK;
}

void arena_put(int dev, Arena a, hipStream_t stream)
{
    a.freed_on = stream;
    a.idle = false;
    DevicePool &P = pool_for(dev);
    bool over = false;
    {
        std::lock_guard<std::mutex> g(P.mu);
        a.seq = ++P.seq;
        P.free_list.push_back(a);
        P.kept += a.bytes;
        over = P.kept > pool_cap_bytes() || P.free_list.size() > kPoolMaxArenas;
    }
    if (over)
        shrink_pool(P);
}

// ------------------------------------------------------- pinned N slots
//
// N goes back to the host through pinned, coherent host memory: on a fresh
// dispatch the layout's count kernel stores it there directly (a
// system-scope store, once, as soon as the counts are known), so no copy is
// enqueued and the host need not wait for the position kernel: it polls the
// slot.  Slots come from a process-wide free list (pages of kSlotsPerPage,
// allocated once, never released) and are held only for the duration of one
// call.

constexpr int64_t kNoValue = INT64_MIN;
constexpr int kSlotsPerPage = 64;

struct Slot {
    int64_t *host = nullptr;  // where the host reads it
    int64_t *dev = nullptr;   // the same memory as the GPU addresses it
};

struct SlotPool {
    std::mutex mu;
    std::vector<Slot> free;
};

SlotPool &slot_pool()
{
    static SlotPool *p = new SlotPool();
    return *p;
}

int slot_get(Slot *out)
{
    SlotPool &P = slot_pool();
    std::lock_guard<std::mutex> g(P.mu);
    if (P.free.empty()) {
        void *page = nullptr;
        hipError_t e = hipHostMalloc(&page, kSlotsPerPage * 64,
                                     hipHostMallocPortable | hipHostMallocCoherent);
        if (e != hipSuccess)
            return hip_fail(e);
        void *dpage = nullptr;
        e = hipHostGetDevicePointer(&dpage, page, 0);
        if (e != hipSuccess) {
            (void)hipHostFree(page);
            return hip_fail(e);
        }
        // one 64-byte line per slot
        for (int i = 0; i < kSlotsPerPage; ++i) {
            Slot sl;
            sl.host = reinterpret_cast<int64_t *>(static_cast<char *>(page) + 64 * i);
            sl.dev = reinterpret_cast<int64_t *>(static_cast<char *>(dpage) + 64 * i);
            P.free.push_back(sl);
        }
    }
    *out = P.free.back();
    P.free.pop_back();
    __atomic_store_n(out->host, kNoValue, __ATOMIC_RELAXED);
    return EP_OK;
}

void slot_put(const Slot &slot)
{
    SlotPool &P = slot_pool();
    std::lock_guard<std::mutex> g(P.mu);
    P.free.push_back(slot);
}

// Waits for the GPU to store a value into the slot.  Every kSlotQueryEvery
// polls (a fraction of a millisecond) it also asks whether the stream is
// still working: a stream that has finished (or failed) without storing one
// ends the wait with an error.  The query is not free: asking every 256 polls
// made the wait for N at 4096 tokens take 28-32 us per call, against
// 13.5-13.9 us asking every 8192 or 65536 polls.
constexpr unsigned kSlotQueryEvery = 16384;

hipError_t slot_wait(const Slot &slot, hipStream_t stream, int64_t *v)
{
    for (unsigned i = 1;; ++i) {
        *v = __atomic_load_n(slot.host, __ATOMIC_ACQUIRE);
        if (*v != kNoValue)
            return hipSuccess;
        if (i % kSlotQueryEvery == 0) {
            const hipError_t q = hipStreamQuery(stream);
            if (q != hipErrorNotReady) {
                *v = __atomic_load_n(slot.host, __ATOMIC_ACQUIRE);
                if (*v != kNoValue)
                    return hipSuccess;
                return q == hipSuccess ? hipErrorUnknown : q;
            }
        }
        __builtin_ia32_pause();
    }
}


// ------------------------------------------------------------ validation

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_dims(const ep_dims *d)
{
    if (d == nullptr)
        return EP_ERR_INVALID;
    if (d->num_tokens < 0 || d->num_tokens > kMaxTokens)
        return EP_ERR_INVALID;
    if (d->hidden <= 0 || d->hidden > kMaxHidden)
        return EP_ERR_INVALID;
    if (d->hidden % 8 != 0)
        return EP_ERR_ALIGN;  // a row must be whole 16-byte vectors
    if (d->num_topk < 1 || d->num_topk > kMaxTopk)
        return EP_ERR_INVALID;
    if (d->num_ranks < 1 || d->num_ranks > kMaxRanks)
        return EP_ERR_INVALID;
    if (d->num_experts < d->num_ranks || d->num_experts > kMaxExperts ||
        d->num_experts % d->num_ranks != 0)
        return EP_ERR_INVALID;
    if (d->num_channels < 1 || d->num_channels > kMaxChannels)
        return EP_ERR_INVALID;
    return EP_OK;
}

int64_t max_rows(const ep_dims &d)
{
    const int64_t km = d.num_topk < d.num_ranks ? d.num_topk : d.num_ranks;
    return int64_t(d.num_tokens) * km;
}

bool same_layout_dims(const ep_dims &a, const ep_dims &b)
{
    return a.num_tokens == b.num_tokens && a.num_topk == b.num_topk &&
           a.num_experts == b.num_experts && a.num_ranks == b.num_ranks &&
           a.num_channels == b.num_channels;
}

}  // namespace

// ---------------------------------------------------------------- handle

struct ep_handle {
    ep_dims dims;
    LayoutShape shape;
    int device = 0;
    Arena arena;
    LayoutBufs bufs;
    std::atomic<int64_t> num_recv{-1};  // N on the host once read back
    std::atomic<bool> dispatched{false};
    bool hashed = false;  // topk_hash[0] holds the hash of the layout's table
    std::atomic<hipStream_t> last_stream{nullptr};
};

namespace {

// EP_CHECK=1: keep a hash of each layout's top-k table and compare it when a
// layout handle comes back with a table (read at every call).
bool check_enabled()
{
    const char *v = std::getenv("EP_CHECK");
    return v != nullptr && v[0] == '1';
}

// Does topk_idx hash to what the handle's layout was made from?  Reads both
// hashes back (synchronizes the stream): a debug check only.
int same_table(ep_handle *h, const int64_t *topk_idx, hipStream_t stream, bool *same);

// Makes a handle and enqueues its layout.  want_n: the caller needs N right
// away; the layout then also stores N into a pinned host slot and this call
// waits for it (the one host synchronization of a fresh dispatch).
int create_handle(const ep_dims &d, const int64_t *topk_idx, const int32_t *rank_mask,
                  hipStream_t stream, bool want_n, ep_handle **out)
{
    ep_handle *h = new (std::nothrow) ep_handle();
    if (h == nullptr)
        return EP_ERR_NOMEM;
    h->dims = d;
    h->shape = layout_shape(d);
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e);
    }
    size_t off[kArenaFields];
    const size_t bytes = layout_arena_bytes(h->shape, off);
    int rc = arena_get(h->device, bytes, stream, &h->arena);
    if (rc != EP_OK) {
        delete h;
        return rc;
    }
    h->bufs = layout_bufs_at(h->arena.ptr, off);
    h->last_stream = stream;
    Slot slot;
    if (want_n) {
        rc = slot_get(&slot);
        if (rc != EP_OK) {
            ep_handle_free(h);
            return rc;
        }
    }
    e = launch_layout(h->shape, topk_idx, rank_mask, h->bufs, slot.dev, h->arena.lc, stream);
    if (e == hipSuccess && check_enabled() && topk_idx != nullptr) {
        e = launch_topk_hash(topk_idx, int64_t(d.num_tokens) * d.num_topk, h->bufs.topk_hash,
                             stream);
        h->hashed = e == hipSuccess;
    }
    if (e != hipSuccess) {
        if (want_n) {
            // a layout kernel enqueued before the failure may still store
            // into the slot: let it finish before the slot is reused
            (void)hipStreamSynchronize(stream);
            slot_put(slot);
        }
        ep_handle_free(h);
        return hip_fail(e);
    }
    if (want_n) {
        // the layout stores N into the slot once.  Two kernels: the count
        // kernel does, and the host polls for it while the positions are
        // still being written.  One launch: N comes at its end, and one
        // stream synchronization was measured faster than polling.
        int64_t n = kNoValue;
        hipError_t e2;
        if (h->shape.fused) {
            e2 = hipStreamSynchronize(stream);
            n = __atomic_load_n(slot.host, __ATOMIC_ACQUIRE);
            if (e2 == hipSuccess && n == kNoValue)
                e2 = hipErrorUnknown;
        } else {
            e2 = slot_wait(slot, stream, &n);
        }
        if (e2 != hipSuccess) {
            // nothing stores into the slot any more: the stream has ended
            (void)hipStreamSynchronize(stream);
            slot_put(slot);
            ep_handle_free(h);
            return hip_fail(e2);
        }
        slot_put(slot);
        h->num_recv.store(n);
    }
    *out = h;
    return EP_OK;
}

int same_table(ep_handle *h, const int64_t *topk_idx, hipStream_t stream, bool *same)
{
    const int64_t n = int64_t(h->dims.num_tokens) * h->dims.num_topk;
    hipError_t e = launch_topk_hash(topk_idx, n, h->bufs.topk_hash + 1, stream);
    uint64_t v[2] = {0, 0};
    if (e == hipSuccess)
        e = hipMemcpyAsync(v, h->bufs.topk_hash, sizeof v, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return hip_fail(e);
    *same = v[0] == v[1];
    return EP_OK;
}

// N of a handle: cached on the host after the first read.  Otherwise it is
// copied from the handle into a pinned slot, which the host polls.
int read_num_recv(ep_handle *h, hipStream_t stream, int64_t *n)
{
    int64_t v = h->num_recv.load();
    if (v < 0) {
        Slot slot;
        int rc = slot_get(&slot);
        if (rc != EP_OK)
            return rc;
        hipError_t e = hipMemcpyAsync(slot.host, h->bufs.num_recv, sizeof(int64_t),
                                      hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess)
            e = slot_wait(slot, stream, &v);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(stream);  // nothing may store into the slot any more
            slot_put(slot);
            return hip_fail(e);
        }
        slot_put(slot);
        h->num_recv.store(v);
    }
    *n = v;
    return EP_OK;
}

// Is a buffer of `cap` rows large enough?  Reads N only when cap is below
// the worst case.
int check_capacity(ep_handle *h, int64_t cap, hipStream_t stream)
{
    if (cap >= max_rows(h->dims))
        return EP_OK;
    int64_t n = 0;
    int rc = read_num_recv(h, stream, &n);
    if (rc != EP_OK)
        return rc;
    return n <= cap ? EP_OK : EP_ERR_CAPACITY;
}

int copy_layout(ep_handle *h, const ep_layout_out *o, hipStream_t stream)
{
    const int64_t T = h->dims.num_tokens, R = h->dims.num_ranks, E = h->dims.num_experts;
    const int64_t C = h->dims.num_channels;
    const void *ptrs[8] = {o->num_tokens_per_rank,   o->num_tokens_per_expert,
                           o->is_token_in_rank,      o->rank_prefix_matrix,
                           o->channel_prefix_matrix, o->recv_channel_prefix_matrix,
                           o->send_head,             o->recv_src_idx};
    for (int i = 0; i < 8; ++i)
        if (ptrs[i] != nullptr && i != 2 && !aligned(ptrs[i], 4))
            return EP_ERR_ALIGN;
    int64_t src_rows = max_rows(h->dims);
    if (o->recv_src_idx != nullptr) {
        if (o->recv_src_cap < 0)
            return EP_ERR_INVALID;
        if (o->recv_src_cap < src_rows) {
            int64_t n = 0;
            int rc = read_num_recv(h, stream, &n);
            if (rc != EP_OK)
                return rc;
            if (n > o->recv_src_cap)
                return EP_ERR_CAPACITY;
            src_rows = n;
        }
    }
    struct Item {
        void *dst;
        const void *src;
        size_t bytes;
    } items[8] = {
        {o->num_tokens_per_rank, h->bufs.num_tokens_per_rank, size_t(R) * 4},
        {o->num_tokens_per_expert, h->bufs.num_tokens_per_expert, size_t(E) * 4},
        {o->is_token_in_rank, h->bufs.is_token_in_rank, size_t(T * R)},
        {o->rank_prefix_matrix, h->bufs.rank_prefix_matrix, size_t(R) * 4},
        {o->channel_prefix_matrix, h->bufs.channel_prefix_matrix, size_t(R * C) * 4},
        {o->recv_channel_prefix_matrix, h->bufs.recv_channel_prefix_matrix, size_t(R * C) * 4},
        {o->send_head, h->bufs.send_head, size_t(T * R) * 4},
        {o->recv_src_idx, h->bufs.recv_src_idx, size_t(src_rows) * 4},
    };
    for (const Item &it : items) {
        if (it.dst == nullptr || it.bytes == 0)
            continue;
        hipError_t e = hipMemcpyAsync(it.dst, it.src, it.bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    h->last_stream = stream;
    return EP_OK;
}

// ------------------------------------------------------ static scratch
//
// The scratch of ep_get_dispatch_layout_noalloc: one static device array per
// GPU (the code object's own memory, no allocation).  Host code never uses
// the array's name as an address: each device's address comes from
// hipGetSymbolAddress, once per device, with that device current.

static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

int scratch_ptr(int dev, void **out)
{
    static std::mutex mu;
    static std::map<int, void *> ptrs;
    std::lock_guard<std::mutex> g(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) {
        *out = it->second;
        return EP_OK;
    }
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
        return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    ptrs[dev] = p;
    *out = p;
    return EP_OK;
}

}  // namespace

// ------------------------------------------------------------------- ABI

extern "C" {

int64_t ep_max_recv_rows(const ep_dims *dims)
{
    if (check_dims(dims) != EP_OK)
        return -1;
    return max_rows(*dims);
}

int ep_get_dispatch_layout(const ep_dims *dims, const int64_t *topk_idx, const int32_t *rank_mask,
                           ep_layout_out *out, ep_handle **handle_out, ep_stream_t stream_)
{
    TraceRange trace_range("ep_get_dispatch_layout");
    try {
        int rc = check_dims(dims);
        if (rc != EP_OK)
            return rc;
        if (dims->num_tokens > 0 && topk_idx == nullptr)
            return EP_ERR_INVALID;
        if (!aligned(topk_idx, 8) || !aligned(rank_mask, 4))
            return EP_ERR_ALIGN;
        if (out == nullptr && handle_out == nullptr)
            return EP_ERR_INVALID;
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        // a recv_src_idx buffer below the worst case needs N for its check
        const bool want_n = out != nullptr && out->recv_src_idx != nullptr &&
                            out->recv_src_cap >= 0 && out->recv_src_cap < max_rows(*dims);
        ep_handle *h = nullptr;
        rc = create_handle(*dims, topk_idx, rank_mask, stream, want_n, &h);
        if (rc != EP_OK)
            return rc;
        if (out != nullptr)
            rc = copy_layout(h, out, stream);
        if (handle_out != nullptr && rc == EP_OK)
            *handle_out = h;
        else
            ep_handle_free(h);
        return rc;
    } catch (const std::bad_alloc &) {
        return EP_ERR_NOMEM;
    } catch (...) {
        return EP_ERR_INVALID;
    }
}

int ep_get_dispatch_layout_noalloc(const ep_dims *dims, const int64_t *topk_idx,
                                   const int32_t *rank_mask, ep_layout_out *out,
                                   ep_stream_t stream_)
{
    TraceRange trace_range("ep_get_dispatch_layout_noalloc");
    try {
        int rc = check_dims(dims);
        if (rc != EP_OK)
            return rc;
        if (out == nullptr || (dims->num_tokens > 0 && topk_idx == nullptr))
            return EP_ERR_INVALID;
        if (!aligned(topk_idx, 8) || !aligned(rank_mask, 4))
            return EP_ERR_ALIGN;
        const void *i32s[6] = {out->num_tokens_per_rank,   out->num_tokens_per_expert,
                               out->rank_prefix_matrix,    out->channel_prefix_matrix,
                               out->recv_channel_prefix_matrix, out->recv_src_idx};
        for (const void *p : i32s)
            if (!aligned(p, 4))
                return EP_ERR_ALIGN;
        if (!aligned(out->send_head, 16) || !aligned(out->is_token_in_rank, 4))
            return EP_ERR_ALIGN;
        if (out->recv_src_idx != nullptr && out->recv_src_cap < max_rows(*dims))
            return EP_ERR_CAPACITY;
        const LayoutShape shape = layout_shape(*dims, false);
        size_t off[kArenaFields];
        if (layout_arena_bytes(shape, off) > size_t(EP_NOALLOC_SCRATCH_BYTES))
            return EP_ERR_TOO_LARGE;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return hip_fail(e);
        void *base = nullptr;
        rc = scratch_ptr(dev, &base);
        if (rc != EP_OK)
            return rc;
        // the kernels write the caller's buffers; fields left NULL go to scratch
        LayoutBufs b = layout_bufs_at(base, off);
        if (out->num_tokens_per_rank != nullptr)
            b.num_tokens_per_rank = out->num_tokens_per_rank;
        if (out->num_tokens_per_expert != nullptr)
            b.num_tokens_per_expert = out->num_tokens_per_expert;
        if (out->is_token_in_rank != nullptr)
            b.is_token_in_rank = out->is_token_in_rank;
        if (out->rank_prefix_matrix != nullptr)
            b.rank_prefix_matrix = out->rank_prefix_matrix;
        if (out->channel_prefix_matrix != nullptr)
            b.channel_prefix_matrix = out->channel_prefix_matrix;
        if (out->recv_channel_prefix_matrix != nullptr)
            b.recv_channel_prefix_matrix = out->recv_channel_prefix_matrix;
        if (out->send_head != nullptr)
            b.send_head = out->send_head;
        if (out->recv_src_idx != nullptr)
            b.recv_src_idx = out->recv_src_idx;
        LayoutCounters unused;  // the multi-kernel path never touches them
        e = launch_layout(shape, topk_idx, rank_mask, b, nullptr, unused,
                          static_cast<hipStream_t>(stream_));
        return e == hipSuccess ? EP_OK : hip_fail(e);
    } catch (...) {
        return EP_ERR_INVALID;
    }
}

int ep_dispatch(const ep_dims *dims, const void *x, const int64_t *topk_idx,
                const float *topk_weights, const int32_t *rank_mask, ep_handle **handle,
                void *recv_x, int64_t *recv_topk_idx, float *recv_topk_weights, int64_t recv_cap,
                int64_t *num_recv, ep_stream_t stream_)
{
    TraceRange trace_range("ep_dispatch");
    try {
        int rc = check_dims(dims);
        if (rc != EP_OK)
            return rc;
        if (handle == nullptr)
            return EP_ERR_INVALID;
        const bool rows = dims->num_tokens > 0;
        if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
            !aligned(recv_topk_idx, 8) || !aligned(topk_weights, 4) ||
            !aligned(recv_topk_weights, 4) || !aligned(rank_mask, 4))
            return EP_ERR_ALIGN;
        if (recv_x != nullptr && x == nullptr && rows)
            return EP_ERR_INVALID;
        if (recv_topk_idx != nullptr && topk_idx == nullptr)
            return EP_ERR_INVALID;
        if (recv_topk_weights != nullptr && (topk_weights == nullptr || topk_idx == nullptr))
            return EP_ERR_INVALID;
        if (recv_cap < 0)
            return EP_ERR_INVALID;
        hipStream_t stream = static_cast<hipStream_t>(stream_);

        ep_handle *h = *handle;
        const bool fresh = h == nullptr;
        if (fresh) {
            if (topk_idx == nullptr && rows)
                return EP_ERR_INVALID;
        } else {
            if (!same_layout_dims(h->dims, *dims))
                return EP_ERR_HANDLE;
            // The mask shapes the layout; a handle already holds one.
            if (rank_mask != nullptr)
                return EP_ERR_INVALID;
            // A handle returned by a dispatch is the cached fast path: the
            // layout is known, so new routing is refused.
            if (h->dispatched.load() && (topk_idx != nullptr || topk_weights != nullptr))
                return EP_ERR_INVALID;
            // A layout handle with its table: under EP_CHECK=1 the table must
            // be the one the layout came from.
            if (topk_idx != nullptr && h->hashed && check_enabled()) {
                bool same = false;
                rc = same_table(h, topk_idx, static_cast<hipStream_t>(stream_), &same);
                if (rc != EP_OK)
                    return rc;
                if (!same)
                    return EP_ERR_INVALID;
            }
        }
        const bool pack = recv_x != nullptr || recv_topk_idx != nullptr || recv_topk_weights != nullptr;
        if (fresh) {
            // N is needed now when the caller asks for it or a buffer is
            // below the worst case: the layout hands it over directly.
            const bool want_n = num_recv != nullptr || (pack && recv_cap < max_rows(*dims));
            rc = create_handle(*dims, topk_idx, rank_mask, stream, want_n, &h);
            if (rc != EP_OK)
                return rc;
        }
        // A handle made here is released again on any error below, so that
        // an error leaves *handle untouched.
        auto fail = [&](int code) {
            if (fresh)
                ep_handle_free(h);
            return code;
        };
        if (pack) {
            rc = check_capacity(h, recv_cap, stream);
            if (rc != EP_OK)
                return fail(rc);
            hipError_t e = launch_dispatch(h->shape, dims->hidden, x, h->bufs, topk_idx,
                                           topk_weights, recv_x, recv_topk_idx,
                                           recv_topk_weights, stream);
            if (e != hipSuccess)
                return fail(hip_fail(e));
            h->dispatched = true;
        }
        h->last_stream = stream;
        if (num_recv != nullptr) {
            int64_t n = 0;
            rc = read_num_recv(h, stream, &n);
            if (rc != EP_OK)
                return fail(rc);
            *num_recv = n;
        }
        if (fresh)
            *handle = h;
        return EP_OK;
    } catch (const std::bad_alloc &) {
        return EP_ERR_NOMEM;
    } catch (...) {
        return EP_ERR_INVALID;
    }
}

int ep_combine(ep_handle *h, int32_t hidden, const void *y, int64_t y_rows,
               const float *recv_topk_weights, const void *bias0, const void *bias1,
               const int32_t *rank_mask, void *out, float *combined_topk_weights,
               ep_stream_t stream_)
{
    TraceRange trace_range("ep_combine");
    try {
        if (h == nullptr)
            return EP_ERR_HANDLE;
        if (hidden <= 0 || hidden > kMaxHidden)
            return EP_ERR_INVALID;
        if (hidden % 8 != 0)
            return EP_ERR_ALIGN;
        if (!aligned(y, 16) || !aligned(out, 16) || !aligned(bias0, 16) || !aligned(bias1, 16) ||
            !aligned(recv_topk_weights, 4) || !aligned(combined_topk_weights, 4) ||
            !aligned(rank_mask, 4))
            return EP_ERR_ALIGN;
        const bool rows = h->dims.num_tokens > 0;
        if (rows && (out == nullptr || y == nullptr))
            return EP_ERR_INVALID;
        if (combined_topk_weights != nullptr && recv_topk_weights == nullptr)
            return EP_ERR_INVALID;
        if (y_rows < 0)
            return EP_ERR_INVALID;
        hipStream_t stream = static_cast<hipStream_t>(stream_);
        int rc = check_capacity(h, y_rows, stream);
        if (rc != EP_OK)
            return rc;
        hipError_t e = launch_combine(h->shape, hidden, y, h->bufs, recv_topk_weights, bias0,
                                      bias1, rank_mask, out, combined_topk_weights, stream);
        if (e != hipSuccess)
            return hip_fail(e);
        h->last_stream = stream;
        return EP_OK;
    } catch (...) {
        return EP_ERR_INVALID;
    }
}

}  // extern "C"

namespace {

int ll_dispatch_common(const ep_dims *dims, int32_t num_slots, const void *x,
                       const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                       void *packed_q, float *packed_scale, int32_t *packed_count,
                       int32_t *src_info, int32_t *topk_slot, ep_stream_t stream_)
{
    if (dims == nullptr)
        return EP_ERR_INVALID;
    ep_dims d = *dims;
    d.num_channels = 1;  // channels do not apply to the low-latency path
    int rc = check_dims(&d);
    if (rc != EP_OK)
        return rc;
    if (num_slots < 1 || num_slots > kMaxLLSlots)
        return EP_ERR_INVALID;
    if (d.num_tokens > num_slots)
        return EP_ERR_CAPACITY;
    if (packed_count == nullptr || src_info == nullptr)
        return EP_ERR_INVALID;
    if (d.num_tokens > 0 && (topk_idx == nullptr || topk_slot == nullptr))
        return EP_ERR_INVALID;
    const bool rows = packed_x != nullptr || packed_q != nullptr;
    if (rows && x == nullptr && d.num_tokens > 0)
        return EP_ERR_INVALID;
    if (packed_q != nullptr && (packed_scale == nullptr || d.hidden % 128 != 0))
        return packed_scale == nullptr ? EP_ERR_INVALID : EP_ERR_ALIGN;
    if (!aligned(x, 16) || !aligned(packed_x, 16) || !aligned(packed_q, 8) ||
        !aligned(packed_scale, 4) || !aligned(topk_idx, 8) || !aligned(rank_mask, 4) ||
        !aligned(packed_count, 4) || !aligned(src_info, 4) || !aligned(topk_slot, 4))
        return EP_ERR_ALIGN;
    hipError_t e = launch_ll_dispatch(d, num_slots, x, topk_idx, rank_mask, packed_x, packed_q,
                                      packed_scale, packed_count, src_info, topk_slot,
                                      static_cast<hipStream_t>(stream_));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int check_lb(const void *a, const void *b, const int64_t *mapping, int32_t num_replicas,
             int32_t num_experts, int64_t elems)
{
    if (num_replicas < 0 || num_replicas > 65535 || num_experts < 1 || elems < 0)
        return EP_ERR_INVALID;
    if (elems % 8 != 0)
        return EP_ERR_ALIGN;
    if (num_replicas > 0 && elems > 0 && (a == nullptr || b == nullptr || mapping == nullptr))
        return EP_ERR_INVALID;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(mapping, 8))
        return EP_ERR_ALIGN;
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_ll_dispatch(const ep_dims *dims, int32_t num_slots, const void *x,
                   const int64_t *topk_idx, const int32_t *rank_mask, void *packed_x,
                   int32_t *packed_count, int32_t *src_info, int32_t *topk_slot,
                   ep_stream_t stream)
{
    TraceRange trace_range("ep_ll_dispatch");
    return ll_dispatch_common(dims, num_slots, x, topk_idx, rank_mask, packed_x, nullptr, nullptr,
                              packed_count, src_info, topk_slot, stream);
}

int ep_ll_dispatch_fp8(const ep_dims *dims, int32_t num_slots, const void *x,
                       const int64_t *topk_idx, const int32_t *rank_mask, void *packed_q,
                       float *packed_scale, int32_t *packed_count, int32_t *src_info,
                       int32_t *topk_slot, ep_stream_t stream)
{
    TraceRange trace_range("ep_ll_dispatch_fp8");
    if (packed_q == nullptr || packed_scale == nullptr)
        return EP_ERR_INVALID;
    return ll_dispatch_common(dims, num_slots, x, topk_idx, rank_mask, nullptr, packed_q,
                              packed_scale, packed_count, src_info, topk_slot, stream);
}

int ep_ll_combine(const ep_dims *dims, int32_t num_slots, const void *packed_y,
                  const int64_t *topk_idx, const float *topk_weights,
                  const int32_t *topk_slot, const int32_t *rank_mask, void *out,
                  ep_stream_t stream_)
{
    TraceRange trace_range("ep_ll_combine");
    if (dims == nullptr)
        return EP_ERR_INVALID;
    ep_dims d = *dims;
    d.num_channels = 1;
    int rc = check_dims(&d);
    if (rc != EP_OK)
        return rc;
    if (num_slots < 1 || num_slots > kMaxLLSlots)
        return EP_ERR_INVALID;
    if (d.num_tokens > num_slots)
        return EP_ERR_CAPACITY;
    if (d.num_tokens > 0 && (packed_y == nullptr || topk_idx == nullptr ||
                             topk_weights == nullptr || topk_slot == nullptr || out == nullptr))
        return EP_ERR_INVALID;
    if (!aligned(packed_y, 16) || !aligned(out, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(topk_slot, 4) || !aligned(rank_mask, 4))
        return EP_ERR_ALIGN;
    hipError_t e = launch_ll_combine(d, num_slots, packed_y, topk_idx, topk_weights, topk_slot,
                                     rank_mask, out, static_cast<hipStream_t>(stream_));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_ll_combine_fp8(const ep_dims *dims, int32_t num_slots, const void *packed_q,
                      const float *packed_scale, const int64_t *topk_idx,
                      const float *topk_weights, const int32_t *topk_slot,
                      const int32_t *rank_mask, void *out, ep_stream_t stream_)
{
    TraceRange trace_range("ep_ll_combine_fp8");
    if (dims == nullptr)
        return EP_ERR_INVALID;
    ep_dims d = *dims;
    d.num_channels = 1;
    int rc = check_dims(&d);
    if (rc != EP_OK)
        return rc;
    if (d.hidden % 128 != 0)
        return EP_ERR_ALIGN;  // whole 128-element scale blocks
    if (num_slots < 1 || num_slots > kMaxLLSlots)
        return EP_ERR_INVALID;
    if (d.num_tokens > num_slots)
        return EP_ERR_CAPACITY;
    if (d.num_tokens > 0 &&
        (packed_q == nullptr || packed_scale == nullptr || topk_idx == nullptr ||
         topk_weights == nullptr || topk_slot == nullptr || out == nullptr))
        return EP_ERR_INVALID;
    if (!aligned(packed_q, 8) || !aligned(packed_scale, 4) || !aligned(out, 16) ||
        !aligned(topk_idx, 8) || !aligned(topk_weights, 4) || !aligned(topk_slot, 4) ||
        !aligned(rank_mask, 4))
        return EP_ERR_ALIGN;
    hipError_t e = launch_ll_combine_fp8(d, num_slots, packed_q, packed_scale, topk_idx,
                                         topk_weights, topk_slot, rank_mask, out,
                                         static_cast<hipStream_t>(stream_));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_mask_update(int32_t *rank_mask, int32_t num_ranks, int32_t rank, int32_t masked,
                   ep_stream_t stream)
{
    if (rank_mask == nullptr || num_ranks < 1 || num_ranks > kMaxRanks || rank < 0 ||
        rank >= num_ranks)
        return EP_ERR_INVALID;
    if (!aligned(rank_mask, 4))
        return EP_ERR_ALIGN;
    hipError_t e = launch_mask_set(rank_mask, num_ranks, rank, masked ? 1 : 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_mask_clean(int32_t *rank_mask, int32_t num_ranks, ep_stream_t stream)
{
    if (rank_mask == nullptr || num_ranks < 1 || num_ranks > kMaxRanks)
        return EP_ERR_INVALID;
    if (!aligned(rank_mask, 4))
        return EP_ERR_ALIGN;
    hipError_t e = launch_mask_set(rank_mask, num_ranks, -1, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_mask_query(const int32_t *rank_mask, int32_t num_ranks, int32_t *host_out,
                  ep_stream_t stream_)
{
    if (rank_mask == nullptr || host_out == nullptr || num_ranks < 1 || num_ranks > kMaxRanks)
        return EP_ERR_INVALID;
    if (!aligned(rank_mask, 4))
        return EP_ERR_ALIGN;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    hipError_t e = hipMemcpyAsync(host_out, rank_mask, size_t(num_ranks) * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_lb_reduce_grads(const void *redundant_grads, void *expert_grads, const int64_t *mapping,
                       int32_t num_replicas, int32_t num_experts, int64_t elems_per_expert,
                       ep_stream_t stream)
{
    TraceRange trace_range("ep_lb_reduce_grads");
    int rc = check_lb(redundant_grads, expert_grads, mapping, num_replicas, num_experts,
                      elems_per_expert);
    if (rc != EP_OK)
        return rc;
    hipError_t e = launch_lb_reduce_grads(redundant_grads, expert_grads, mapping, num_replicas,
                                          num_experts, elems_per_expert,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_lb_prefetch_weights(const void *expert_weights, void *redundant_weights,
                           const int64_t *mapping, int32_t num_replicas, int32_t num_experts,
                           int64_t elems_per_expert, ep_stream_t stream)
{
    TraceRange trace_range("ep_lb_prefetch_weights");
    int rc = check_lb(expert_weights, redundant_weights, mapping, num_replicas, num_experts,
                      elems_per_expert);
    if (rc != EP_OK)
        return rc;
    hipError_t e = launch_lb_prefetch_weights(expert_weights, redundant_weights, mapping,
                                              num_replicas, num_experts, elems_per_expert,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? EP_OK : hip_fail(e);
}

int ep_handle_copy_layout(ep_handle *h, ep_layout_out *out, ep_stream_t stream)
{
    if (h == nullptr)
        return EP_ERR_HANDLE;
    if (out == nullptr)
        return EP_ERR_INVALID;
    try {
        return copy_layout(h, out, static_cast<hipStream_t>(stream));
    } catch (...) {
        return EP_ERR_INVALID;
    }
}

int ep_handle_num_recv(ep_handle *h, int64_t *num_recv)
{
    if (h == nullptr)
        return EP_ERR_HANDLE;
    if (num_recv == nullptr)
        return EP_ERR_INVALID;
    return read_num_recv(h, h->last_stream.load(), num_recv);
}

int ep_handle_dims(const ep_handle *h, ep_dims *dims)
{
    if (h == nullptr)
        return EP_ERR_HANDLE;
    if (dims == nullptr)
        return EP_ERR_INVALID;
    *dims = h->dims;
    return EP_OK;
}

size_t ep_handle_nbytes(const ep_handle *h) { return h == nullptr ? 0 : h->arena.bytes; }

void ep_handle_free(ep_handle *h)
{
    if (h == nullptr)
        return;
    int cur = 0;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != h->device;
    if (switch_dev)
        (void)hipSetDevice(h->device);
    arena_put(h->device, h->arena, h->last_stream.load());
    if (switch_dev)
        (void)hipSetDevice(cur);
    delete h;
}

int ep_pool_trim(void)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    return trim_pool(pool_for(dev));
}

int ep_pool_stats(size_t *kept_bytes, int32_t *kept_arenas, size_t *cap_bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    DevicePool &P = pool_for(dev);
    std::lock_guard<std::mutex> g(P.mu);
    if (kept_bytes != nullptr)
        *kept_bytes = P.kept;
    if (kept_arenas != nullptr)
        *kept_arenas = int32_t(P.free_list.size());
    if (cap_bytes != nullptr)
        *cap_bytes = pool_cap_bytes();
    return EP_OK;
}

int ep_set_tuning(const char *op, int a, int b, int c)
{
    if (op == nullptr)
        return EP_ERR_INVALID;
    if (std::strcmp(op, "dispatch") == 0)
        return set_dispatch_tuning(a, b, c) ? EP_OK : EP_ERR_INVALID;
    if (std::strcmp(op, "combine") == 0)
        return set_combine_tuning(a, b, c) ? EP_OK : EP_ERR_INVALID;
    if (std::strcmp(op, "ll") == 0) {
        if (a == -1 && b == -1 && c == -1)
            return set_ll_tuning(0) ? EP_OK : EP_ERR_INVALID;
        return (b == 0 && c == 0 && set_ll_tuning(a)) ? EP_OK : EP_ERR_INVALID;
    }
    if (std::strcmp(op, "layout") == 0) {
        if (a == -1 && b == -1 && c == -1)
            return set_layout_tuning(0) ? EP_OK : EP_ERR_INVALID;
        return (b == 0 && c == 0 && set_layout_tuning(a)) ? EP_OK : EP_ERR_INVALID;
    }
    return EP_ERR_INVALID;
}

int ep_tuning_list(const char *op, int index, int *a, int *b, int *c)
{
    if (op == nullptr || a == nullptr || b == nullptr || c == nullptr)
        return -1;
    if (std::strcmp(op, "dispatch") == 0) {
        const int n = dispatch_tuning_count();
        if (index >= 0 && index < n)
            dispatch_tuning_at(index, a, b, c);
        return n;
    }
    if (std::strcmp(op, "combine") == 0) {
        const int n = combine_tuning_count();
        if (index >= 0 && index < n)
            combine_tuning_at(index, a, b, c);
        return n;
    }
    if (std::strcmp(op, "ll") == 0 || std::strcmp(op, "layout") == 0) {
        if (index >= 0 && index < 3) {
            *a = index;
            *b = 0;
            *c = 0;
        }
        return 3;
    }
    return -1;
}

const char *ep_status_str(int status)
{
    switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID: return "invalid argument";
    case EP_ERR_ALIGN: return "alignment rule broken (16-byte rows and pointers)";
    case EP_ERR_CAPACITY: return "output buffer has too few rows";
    case EP_ERR_HANDLE: return "handle missing or does not match the dims";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_NOMEM: return "out of memory";
    case EP_ERR_TOO_LARGE: return "problem needs more than the no-allocation layout's static scratch";
    default: return "unknown status";
    }
}

const char *ep_last_hip_error(void) { return g_last_hip.c_str(); }

int ep_version(void) { return (2 << 16) | 4; }

}  // extern "C"

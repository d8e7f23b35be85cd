// Adapter residency: a cache of adapters in a caller-owned HBM buffer, filled
// from pinned host copies by asynchronous copies on a copy stream.
//
// The pages ("Multi-LoRA Serving: Many Adapters on One GPU" (gpusmith.com),
// section "Swap latency and cache policy"; "Multi-LoRA Serving in Production
// ..." (llms.blog), sections "Tiered Storage Hierarchy and Asynchronous
// Streaming" and "Eviction and Replacement Policies") describe the tiers: GPU
// slots that a batch can use at once, a host RAM tier one PCIe copy away, and
// storage beyond.  Copies of uncached adapters run on a dedicated copy stream
// while the GPU computes earlier work; when HBM is full the least recently
// used adapter is evicted, and pinned adapters never are.  This file covers
// the GPU and host tiers.
//
// Device buffer: [pool_A u64 x N][pool_B u64 x N][rank i32 x N][alpha f32 x N]
// (the tables the kernels read, indexed by adapter id), then the adapter
// extents.  A resident adapter owns one extent: A [r, d_in] then B [d_out, r],
// each 256-byte aligned and unpadded in rank.  Free space is a list of extents
// kept sorted and merged; placement is first fit.
//
// Ordering (all on the caller's streams, no host synchronisation):
//  * prepare(batch k) first records event E_k on the compute stream: it marks
//    the end of every batch enqueued before k.
//  * An adapter last used by batch j may be overwritten once E_{j+1} has
//    completed, so before copying into freed space the copy stream waits for
//    that event (or for E_k when j is older than the event ring).
//  * The batch's copies and the table update go to the copy stream, whose
//    completion event the compute stream then waits for.  Batches that need no
//    copy add no wait.
//
// The copies are one gather-copy kernel per batch: its workgroups read the
// registered pinned host memory over PCIe and write the extents, 64 KB each,
// so a batch of many small adapters costs one launch instead of two copy
// commands per adapter.  Host memory that the device cannot address directly
// (not pinned, or mapped at another address) is copied with hipMemcpyAsync.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

namespace lora {
namespace {

constexpr size_t kAlign = 256;
constexpr int kStageRing = 4;  // pinned table staging buffers in flight
constexpr int kEventRing = 64; // batch-start events kept

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Extent {
    size_t off, len; // offsets from the start of the data region
};

struct AdapterRec {
    const void *A_host = nullptr;
    const void *B_host = nullptr;
    bool direct = false; // A_host and B_host are pinned and mapped at the same address on the device
    int32_t rank = 0;
    float alpha = 0.f;
    bool registered = false;
    bool resident = false;
    bool pinned = false;
    size_t off = 0, len = 0; // extent while resident
    int64_t last_use = -1;   // batch index
    int64_t mark = -1;       // prepare call that last listed it (duplicate filter)
    int64_t evict_mark = -1; // prepare call whose placement chose it as a victim
};

// One gather-copy launch: entries (source, destination, bytes), each cut
// into kCopyChunk-byte pieces, one workgroup per piece.
constexpr int kCopyEntries = 96;
constexpr uint64_t kCopyChunk = 64u << 10;
struct CopyEntry {
    const uint8_t *src;
    uint8_t *dst;
    uint64_t bytes;
};
struct CopyList {
    CopyEntry e[kCopyEntries];
    int32_t first[kCopyEntries + 1]; // first piece of entry i; first[n] = pieces in all
    int32_t n;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void cache_copy_kernel(const CopyList L)
{
    // the entry of this piece: the last i with first[i] <= blockIdx.x
    const int b = int(blockIdx.x);
    int lo = 0, hi = L.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (L.first[mid] <= b) lo = mid;
        else hi = mid - 1;
    }
    const uint8_t *src = L.e[lo].src;
    uint8_t *dst = L.e[lo].dst;
    const uint64_t off0 = uint64_t(b - L.first[lo]) * kCopyChunk;
    const uint64_t end = L.e[lo].bytes < off0 + kCopyChunk ? L.e[lo].bytes : off0 + kCopyChunk;
    const uint64_t tid = threadIdx.x;
    uint64_t tail = off0;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0) {
        // 16-byte pieces, four in flight per thread
        const uint64_t vend = off0 + ((end - off0) & ~uint64_t(15));
        for (uint64_t base = off0; base < vend; base += 4 * 4096) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t o = base + uint64_t(u) * 4096 + 16 * tid;
                if (o < vend) v[u] = *reinterpret_cast<const u32x4 *>(src + o);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t o = base + uint64_t(u) * 4096 + 16 * tid;
                if (o < vend) *reinterpret_cast<u32x4 *>(dst + o) = v[u];
            }
        }
        tail = vend;
    }
    for (uint64_t o = tail + tid; o < end; o += 256) dst[o] = src[o];
}

// Pinned host memory that the device reads at the same address.
bool device_readable(const void *p)
{
    hipPointerAttribute_t at{};
    const hipError_t e = hipPointerGetAttributes(&at, p);
    if (e != hipSuccess) {
        (void)hipGetLastError(); // a pageable pointer is not an error of the next call
        return false;
    }
    return at.type == hipMemoryTypeHost && at.devicePointer != nullptr && at.devicePointer == at.hostPointer;
}

} // namespace
} // namespace lora

struct lora_cache {
    char *dev = nullptr;
    size_t dev_bytes = 0;
    bool dry = false;
    int32_t n = 0, dtype = 0, d_in = 0, d_out = 0, es = 0;
    size_t tab_bytes = 0, data_bytes = 0;
    std::vector<lora::AdapterRec> ad;
    std::vector<lora::Extent> free_list;
    std::vector<uint64_t> tA, tB;
    std::vector<int32_t> tr;
    std::vector<float> ta;
    void *stage[lora::kStageRing] = {};
    bool stage_direct = false;
    hipEvent_t stage_ev[lora::kStageRing] = {};
    bool stage_busy[lora::kStageRing] = {};
    int stage_next = 0;
    hipEvent_t batch_ev[lora::kEventRing] = {};
    hipEvent_t copy_ev = nullptr;
    int64_t batch = 0; // successful prepare calls (batch index)
    int64_t call = 0;  // every prepare call, failed ones included
    lora_cache_stats st{};
};

namespace lora {
namespace {

size_t extent_bytes(const lora_cache *c, int32_t r)
{
    return round_up(size_t(r) * size_t(c->d_in) * size_t(c->es), kAlign) +
           round_up(size_t(c->d_out) * size_t(r) * size_t(c->es), kAlign);
}

// First fit in free list `fl`; returns false when no free extent is large enough.
bool take(std::vector<Extent> &fl, size_t len, size_t *off)
{
    for (size_t i = 0; i < fl.size(); ++i) {
        Extent &e = fl[i];
        if (e.len < len) continue;
        *off = e.off;
        e.off += len;
        e.len -= len;
        if (e.len == 0) fl.erase(fl.begin() + long(i));
        return true;
    }
    return false;
}

void give_back(std::vector<Extent> &fl, size_t off, size_t len)
{
    auto it = std::lower_bound(fl.begin(), fl.end(), off, [](const Extent &e, size_t o) { return e.off < o; });
    it = fl.insert(it, Extent{off, len});
    // merge with the next, then with the previous extent
    if (it + 1 != fl.end() && it->off + it->len == (it + 1)->off) {
        it->len += (it + 1)->len;
        fl.erase(it + 1);
    }
    if (it != fl.begin() && (it - 1)->off + (it - 1)->len == it->off) {
        (it - 1)->len += it->len;
        fl.erase(it);
    }
}

void set_table(lora_cache *c, int32_t a)
{
    const AdapterRec &r = c->ad[size_t(a)];
    if (r.resident) {
        const uint64_t base = reinterpret_cast<uint64_t>(c->dev) + c->tab_bytes + r.off;
        c->tA[size_t(a)] = base;
        c->tB[size_t(a)] = base + round_up(size_t(r.rank) * size_t(c->d_in) * size_t(c->es), kAlign);
        c->tr[size_t(a)] = r.rank;
        c->ta[size_t(a)] = r.alpha;
    } else {
        c->tA[size_t(a)] = c->tB[size_t(a)] = 0;
        c->tr[size_t(a)] = 0;
        c->ta[size_t(a)] = 0.f;
    }
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

} // namespace
} // namespace lora

using namespace lora;

extern "C" {

size_t lora_cache_table_bytes(int32_t n_adapters)
{
    if (n_adapters < 0) return 0;
    return round_up(size_t(n_adapters) * (8 + 8 + 4 + 4), kAlign);
}

int lora_cache_create(void *dev_buf, size_t dev_bytes, int32_t n_adapters, int dtype, int32_t d_in, int32_t d_out,
                      unsigned flags, lora_cache **out)
{
    clear_error();
    if (!out) return fail(LORA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (dtype != LORA_F32 && dtype != LORA_BF16) return fail(LORA_ERR_DTYPE, "unknown dtype %d", dtype);
    if (n_adapters < 1) return fail(LORA_ERR_ARG, "n_adapters %d < 1", n_adapters);
    if (d_in < 1 || d_out < 1) return fail(LORA_ERR_ARG, "d_in %d, d_out %d must be >= 1", d_in, d_out);
    if (flags & ~unsigned(LORA_CACHE_DRY)) return fail(LORA_ERR_ARG, "unknown flags 0x%x", flags);
    if (!dev_buf) return fail(LORA_ERR_ARG, "dev_buf is NULL");
    if (reinterpret_cast<uintptr_t>(dev_buf) % kAlign) return fail(LORA_ERR_ALIGN, "dev_buf is not 256-byte aligned");
    const size_t tab = lora_cache_table_bytes(n_adapters);
    if (dev_bytes < tab + kAlign)
        return fail(LORA_ERR_WORKSPACE, "buffer %zu B holds no adapter after %zu B of tables", dev_bytes, tab);
    auto *c = new lora_cache();
    c->dev = static_cast<char *>(dev_buf);
    c->dev_bytes = dev_bytes;
    c->dry = (flags & LORA_CACHE_DRY) != 0;
    c->n = n_adapters;
    c->dtype = dtype;
    c->d_in = d_in;
    c->d_out = d_out;
    c->es = dtype == LORA_BF16 ? 2 : 4;
    c->tab_bytes = tab;
    c->data_bytes = (dev_bytes - tab) / kAlign * kAlign;
    c->ad.resize(size_t(n_adapters));
    c->free_list.push_back(Extent{0, c->data_bytes});
    c->tA.assign(size_t(n_adapters), 0);
    c->tB.assign(size_t(n_adapters), 0);
    c->tr.assign(size_t(n_adapters), 0);
    c->ta.assign(size_t(n_adapters), 0.f);
    if (!c->dry) {
        hipError_t e = hipSuccess;
        for (int i = 0; i < kStageRing && e == hipSuccess; ++i) {
            e = hipHostMalloc(&c->stage[i], tab, hipHostMallocDefault);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming);
        }
        for (int i = 0; i < kEventRing && e == hipSuccess; ++i)
            e = hipEventCreateWithFlags(&c->batch_ev[i], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->copy_ev, hipEventDisableTiming);
        if (e == hipSuccess) {
            c->stage_direct = true;
            for (int i = 0; i < kStageRing; ++i) c->stage_direct = c->stage_direct && device_readable(c->stage[i]);
        }
        // tables start out all zero (no adapter resident)
        if (e == hipSuccess) e = hipMemset(c->dev, 0, tab);
        if (e != hipSuccess) {
            lora_cache_destroy(c);
            return hip_fail(e, "lora_cache_create");
        }
    }
    *out = c;
    return LORA_OK;
}

void lora_cache_destroy(lora_cache *c)
{
    if (!c) return;
    if (!c->dry) {
        // copies from the staging buffers may still be in flight
        for (int i = 0; i < kStageRing; ++i) {
            if (c->stage_ev[i]) {
                if (c->stage_busy[i]) (void)hipEventSynchronize(c->stage_ev[i]);
                (void)hipEventDestroy(c->stage_ev[i]);
            }
            if (c->stage[i]) (void)hipHostFree(c->stage[i]);
        }
        for (int i = 0; i < kEventRing; ++i)
            if (c->batch_ev[i]) (void)hipEventDestroy(c->batch_ev[i]);
        if (c->copy_ev) (void)hipEventDestroy(c->copy_ev);
    }
    delete c;
}

int lora_cache_register(lora_cache *c, int32_t adapter, const void *A_host, const void *B_host, int32_t rank,
                        float alpha)
{
    clear_error();
    if (!c) return fail(LORA_ERR_ARG, "cache is NULL");
    if (adapter < 0 || adapter >= c->n) return fail(LORA_ERR_ADAPTER_ID, "adapter %d outside [0, %d)", adapter, c->n);
    if (rank < 1 || rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "rank %d outside [1, 256]", rank);
    if (!A_host || !B_host) return fail(LORA_ERR_ARG, "A_host or B_host is NULL");
    AdapterRec &r = c->ad[size_t(adapter)];
    if (r.resident) return fail(LORA_ERR_ARG, "adapter %d is resident; it cannot be registered again", adapter);
    r.A_host = A_host;
    r.B_host = B_host;
    r.direct = !c->dry && device_readable(A_host) && device_readable(B_host);
    r.rank = rank;
    r.alpha = alpha;
    r.registered = true;
    return LORA_OK;
}

int lora_cache_pin(lora_cache *c, int32_t adapter, int pinned)
{
    clear_error();
    if (!c) return fail(LORA_ERR_ARG, "cache is NULL");
    if (adapter < 0 || adapter >= c->n) return fail(LORA_ERR_ADAPTER_ID, "adapter %d outside [0, %d)", adapter, c->n);
    c->ad[size_t(adapter)].pinned = pinned != 0;
    return LORA_OK;
}

int lora_cache_prepare(lora_cache *c, const int32_t *ids_host, int32_t T, void *copy_stream, void *compute_stream)
{
    clear_error();
    if (!c) return fail(LORA_ERR_ARG, "cache is NULL");
    if (T < 0) return fail(LORA_ERR_ARG, "T %d < 0", T);
    if (T > 0 && !ids_host) return fail(LORA_ERR_ARG, "ids_host is NULL");
    const int64_t k = c->batch;
    // a fresh mark per call: marks left by a call that failed must not hide
    // adapters from the next one
    const int64_t m = ++c->call;
    // the batch's distinct adapters, in first-appearance order
    static thread_local std::vector<int32_t> used;
    used.clear();
    for (int32_t t = 0; t < T; ++t) {
        const int32_t a = ids_host[t];
        if (a == -1) continue;
        if (a < -1 || a >= c->n) return fail(LORA_ERR_ADAPTER_ID, "ids[%d] = %d outside [-1, %d)", t, a, c->n);
        AdapterRec &r = c->ad[size_t(a)];
        if (!r.registered) return fail(LORA_ERR_ADAPTER_ID, "adapter %d is not registered", a);
        if (r.mark != m) {
            r.mark = m;
            used.push_back(a);
        }
    }
    // the whole batch must fit next to the pinned adapters it does not use
    size_t need = 0, pinned_other = 0;
    for (int32_t a : used) need += extent_bytes(c, c->ad[size_t(a)].rank);
    for (const AdapterRec &r : c->ad)
        if (r.resident && r.pinned && r.mark != m) pinned_other += r.len;
    if (need + pinned_other > c->data_bytes)
        return fail(LORA_ERR_WORKSPACE, "batch needs %zu B of adapters; the cache holds %zu B (%zu B pinned)", need,
                    c->data_bytes, pinned_other);

    // Placement, on a scratch copy of the free list: every miss gets an
    // extent, evicting least recently used adapters that are neither pinned
    // nor in this batch.  Nothing of the cache changes until every miss has
    // its place, so a batch that cannot be placed leaves the cache as it was.
    static thread_local std::vector<Extent> fl;
    static thread_local std::vector<int32_t> victims;
    static thread_local std::vector<std::pair<int32_t, size_t>> placed;
    fl = c->free_list;
    victims.clear();
    placed.clear();
    for (int32_t a : used) {
        const AdapterRec &r = c->ad[size_t(a)];
        if (r.resident) continue;
        const size_t len = extent_bytes(c, r.rank);
        size_t off = 0;
        while (!take(fl, len, &off)) {
            int32_t victim = -1;
            for (int32_t b = 0; b < c->n; ++b) {
                const AdapterRec &q = c->ad[size_t(b)];
                if (!q.resident || q.pinned || q.mark == m || q.evict_mark == m) continue;
                if (victim < 0 || q.last_use < c->ad[size_t(victim)].last_use) victim = b;
            }
            if (victim < 0)
                return fail(LORA_ERR_WORKSPACE, "no evictable adapter leaves %zu contiguous bytes for adapter %d "
                            "(fragmented cache)", len, a);
            AdapterRec &q = c->ad[size_t(victim)];
            q.evict_mark = m;
            give_back(fl, q.off, q.len);
            victims.push_back(victim);
        }
        placed.emplace_back(a, off);
    }

    hipStream_t cs = static_cast<hipStream_t>(compute_stream), xs = static_cast<hipStream_t>(copy_stream);
    hipEvent_t start_ev = nullptr;
    if (!c->dry) {
        start_ev = c->batch_ev[k % kEventRing];
        hipError_t e = hipEventRecord(start_ev, cs);
        if (e != hipSuccess) return hip_fail(e, "lora_cache_prepare: event record");
    }
    // commit the placement
    c->free_list.swap(fl);
    int64_t wait_batch = -1; // newest batch whose reads an overwrite must follow
    for (int32_t v : victims) {
        AdapterRec &q = c->ad[size_t(v)];
        q.resident = false;
        wait_batch = std::max(wait_batch, q.last_use);
        c->st.resident_bytes -= int64_t(q.len);
        --c->st.resident;
        ++c->st.evictions;
        set_table(c, v);
    }
    static thread_local std::vector<int32_t> loads;
    loads.clear();
    for (const auto &pa : placed) {
        AdapterRec &r = c->ad[size_t(pa.first)];
        r.resident = true;
        r.off = pa.second;
        r.len = extent_bytes(c, r.rank);
        c->st.resident_bytes += int64_t(r.len);
        ++c->st.resident;
        ++c->st.misses;
        set_table(c, pa.first);
        loads.push_back(pa.first);
    }
    c->st.hits += int64_t(used.size() - placed.size());
    for (int32_t a : used) c->ad[size_t(a)].last_use = k;
    ++c->st.batches;
    c->batch = k + 1;
    if (loads.empty() || c->dry) {
        for (int32_t a : loads) {
            const AdapterRec &r = c->ad[size_t(a)];
            c->st.bytes_copied += int64_t(size_t(r.rank) * size_t(c->d_in + c->d_out) * size_t(c->es));
        }
        return LORA_OK;
    }
    hipError_t e = hipSuccess;
    // space freed from an adapter that batch j read is rewritten only after
    // batch j's kernels: the event recorded at the start of batch j + 1
    if (wait_batch >= 0) {
        const hipEvent_t w = (wait_batch + 1 < k && k - (wait_batch + 1) < kEventRing)
                                 ? c->batch_ev[(wait_batch + 1) % kEventRing]
                                 : start_ev;
        e = hipStreamWaitEvent(xs, w, 0);
    }
    CopyList L{};
    int32_t pieces = 0;
    auto flush = [&]() -> hipError_t {
        if (L.n == 0) return hipSuccess;
        L.first[L.n] = pieces;
        hipLaunchKernelGGL(cache_copy_kernel, dim3(unsigned(pieces)), dim3(256), 0, xs, L);
        const hipError_t le = hipGetLastError();
        L.n = 0;
        pieces = 0;
        return le;
    };
    auto add = [&](const void *src, void *dst, uint64_t bytes) -> hipError_t {
        hipError_t fe = hipSuccess;
        if (L.n == kCopyEntries) fe = flush();
        L.e[L.n] = CopyEntry{static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), bytes};
        L.first[L.n] = pieces;
        pieces += int32_t((bytes + kCopyChunk - 1) / kCopyChunk);
        ++L.n;
        return fe;
    };
    for (size_t i = 0; i < loads.size() && e == hipSuccess; ++i) {
        const AdapterRec &r = c->ad[size_t(loads[i])];
        const size_t a_bytes = size_t(r.rank) * size_t(c->d_in) * size_t(c->es);
        const size_t b_bytes = size_t(c->d_out) * size_t(r.rank) * size_t(c->es);
        char *dst = c->dev + c->tab_bytes + r.off;
        if (r.direct) {
            e = add(r.A_host, dst, a_bytes);
            if (e == hipSuccess) e = add(r.B_host, dst + round_up(a_bytes, kAlign), b_bytes);
        } else {
            e = hipMemcpyAsync(dst, r.A_host, a_bytes, hipMemcpyHostToDevice, xs);
            if (e == hipSuccess) e = hipMemcpyAsync(dst + round_up(a_bytes, kAlign), r.B_host, b_bytes,
                                                    hipMemcpyHostToDevice, xs);
        }
        c->st.bytes_copied += int64_t(a_bytes + b_bytes);
    }
    // tables: staged in pinned memory (a ring, so that a buffer is rewritten
    // only after its previous copy has run) and copied after the adapters
    if (e == hipSuccess) {
        const int s = c->stage_next;
        c->stage_next = (s + 1) % kStageRing;
        if (c->stage_busy[s]) e = hipEventSynchronize(c->stage_ev[s]);
        if (e == hipSuccess) {
            char *p = static_cast<char *>(c->stage[s]);
            const size_t n = size_t(c->n);
            std::memcpy(p, c->tA.data(), 8 * n);
            std::memcpy(p + 8 * n, c->tB.data(), 8 * n);
            std::memcpy(p + 16 * n, c->tr.data(), 4 * n);
            std::memcpy(p + 20 * n, c->ta.data(), 4 * n);
            if (c->stage_direct) {
                e = add(p, c->dev, 24 * n);
                if (e == hipSuccess) e = flush();
            } else {
                e = flush();
                if (e == hipSuccess) e = hipMemcpyAsync(c->dev, p, 24 * n, hipMemcpyHostToDevice, xs);
            }
        }
        if (e == hipSuccess) e = hipEventRecord(c->stage_ev[s], xs);
        if (e == hipSuccess) c->stage_busy[s] = true;
    }
    if (e == hipSuccess) e = hipEventRecord(c->copy_ev, xs);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, c->copy_ev, 0);
    if (e != hipSuccess) {
        // the batch's copies were not all enqueued: its misses are not resident
        for (int32_t a : loads) {
            AdapterRec &r = c->ad[size_t(a)];
            r.resident = false;
            give_back(c->free_list, r.off, r.len);
            c->st.resident_bytes -= int64_t(r.len);
            --c->st.resident;
            set_table(c, a);
        }
        return hip_fail(e, "lora_cache_prepare: copies");
    }
    return LORA_OK;
}

int lora_cache_view_get(const lora_cache *c, lora_cache_view *out)
{
    clear_error();
    if (!c || !out) return fail(LORA_ERR_ARG, "cache or out is NULL");
    const size_t n = size_t(c->n);
    out->pool_A_dev = reinterpret_cast<const uint64_t *>(c->dev);
    out->pool_B_dev = reinterpret_cast<const uint64_t *>(c->dev + 8 * n);
    out->rank_dev = reinterpret_cast<const int32_t *>(c->dev + 16 * n);
    out->alpha_dev = reinterpret_cast<const float *>(c->dev + 20 * n);
    out->pool_A_host = c->tA.data();
    out->pool_B_host = c->tB.data();
    out->rank_host = c->tr.data();
    out->alpha_host = c->ta.data();
    out->n_adapters = c->n;
    int32_t mr = 0;
    for (const AdapterRec &r : c->ad)
        if (r.registered && r.rank > mr) mr = r.rank;
    out->max_rank = mr;
    return LORA_OK;
}

int lora_cache_stats_get(const lora_cache *c, lora_cache_stats *out)
{
    clear_error();
    if (!c || !out) return fail(LORA_ERR_ARG, "cache or out is NULL");
    *out = c->st;
    return LORA_OK;
}

} // extern "C"

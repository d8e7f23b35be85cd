// C ABI entry points: argument checks, the host-side plan builder, dispatch to
// the kernel launchers.  Nothing here touches device memory except through
// hipMemcpyAsync (plan upload) and kernel launches on the caller's stream.
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

#include <cmath>

static_assert(sizeof(lora_blk_desc) == 128, "block descriptor is one 128-byte record");
static_assert(sizeof(lora_seg_desc) == 40, "segment descriptor layout");
static_assert(sizeof(lora_chunk_desc) == 320, "chunk descriptor layout");
static_assert(sizeof(lora_plan_header) == 96, "plan header layout");

namespace lora {

static thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

LaunchEvents &launch_events()
{
    static thread_local LaunchEvents le;
    return le;
}

static size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// The segment table as arrays, at the plan's soa_offset: seg_A[S], seg_B[S]
// (uint64), seg_indptr[S + 1], seg_adapter[S], seg_rank[S] (int32),
// seg_scale[S] (float).
struct SoA {
    uint64_t *A, *B;
    int32_t *indptr, *adapter, *rank;
    float *scale;
};
static size_t soa_bytes(int32_t S) { return 16 * size_t(S) + 4 * (size_t(S) + 1) + 12 * size_t(S); }
static SoA soa_at(char *p, int32_t S)
{
    SoA t;
    t.A = reinterpret_cast<uint64_t *>(p);
    t.B = t.A + S;
    t.indptr = reinterpret_cast<int32_t *>(t.B + S);
    t.adapter = t.indptr + S + 1;
    t.rank = t.adapter + S;
    t.scale = reinterpret_cast<float *>(t.rank + S);
    return t;
}

static int esize_of(int dtype) { return dtype == LORA_BF16 ? 2 : 4; }

static bool elem_aligned(const void *p, int es)
{
    return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(es)) == 0;
}

// Validates a host buffer holding a built plan and returns its header.
static int check_plan(const void *plan_host, const lora_plan_header **out)
{
    if (!plan_host) return fail(LORA_ERR_ARG, "the segments' host buffer is NULL");
    if (reinterpret_cast<uintptr_t>(plan_host) & 7u)
        return fail(LORA_ERR_ALIGN, "the segments' host buffer is not 8-byte aligned");
    const auto *h = static_cast<const lora_plan_header *>(plan_host);
    if (h->magic != LORA_PLAN_MAGIC) return fail(LORA_ERR_PLAN, "plan buffer holds no built plan");
    if (h->num_segments < 0 || h->num_sorted < 0 || h->num_blocks < 0 ||
        h->num_sorted > h->num_tokens || h->max_rank < 0 || h->max_rank > LORA_MAX_RANK)
        return fail(LORA_ERR_PLAN, "plan header is inconsistent");
    *out = h;
    return LORA_OK;
}

// Validates a device segments struct: the header comes from its host copy
// (launch geometry), *dev is the device copy the kernels read.
static int check_segments(const lora_segments *seg, const lora_plan_header **h, const char **dev)
{
    if (!seg) return fail(LORA_ERR_ARG, "segments is NULL");
    if (!seg->host) return fail(LORA_ERR_ARG, "segments have no host copy (not uploaded with lora_segments_upload)");
    const int st = check_plan(seg->host, h);
    if (st) return st;
    *dev = static_cast<const char *>(seg->buf);
    return LORA_OK;
}

static int check_dtype(int dtype)
{
    if (dtype != LORA_F32 && dtype != LORA_BF16) return fail(LORA_ERR_DTYPE, "unknown dtype %d", dtype);
    return LORA_OK;
}

static int check_v(const float *v, int64_t ldv, int32_t max_rank)
{
    if (!v) return fail(LORA_ERR_ARG, "v is NULL");
    if (!aligned16(v)) return fail(LORA_ERR_ALIGN, "v is not 16-byte aligned");
    if (ldv < max_rank || ldv < 1) return fail(LORA_ERR_RANK, "ldv %lld < max rank %d", (long long)ldv, max_rank);
    if (ldv % 4) return fail(LORA_ERR_ALIGN, "ldv %lld is not a multiple of 4", (long long)ldv);
    return LORA_OK;
}

// Shared checks of x / d_in for both shrink flavours; fills ShrinkArgs.
static int make_shrink_args(int dtype, const void *x, int64_t ldx, int32_t d_in, float *v, int64_t ldv,
                            int32_t max_rank, ShrinkArgs *sa)
{
    int st = check_dtype(dtype);
    if (st) return st;
    if (!x) return fail(LORA_ERR_ARG, "x is NULL");
    if (d_in < 1) return fail(LORA_ERR_ARG, "d_in %d < 1", d_in);
    if (ldx < d_in) return fail(LORA_ERR_ARG, "ldx %lld < d_in %d", (long long)ldx, d_in);
    const int es = esize_of(dtype);
    if (!elem_aligned(x, es)) return fail(LORA_ERR_ALIGN, "x is not aligned to its element size");
    if ((st = check_v(v, ldv, max_rank))) return st;
    sa->dtype = dtype;
    sa->x = x;
    sa->ldx = ldx;
    sa->d_in = d_in;
    sa->v = v;
    sa->ldv = ldv;
    // 16-byte row loads need aligned x rows and A rows (A_i row pitch = d_in).
    sa->vec = aligned16(x) && ((ldx * es) % 16 == 0) && ((int64_t(d_in) * es) % 16 == 0);
    return LORA_OK;
}

static int make_expand_args(int dtype, const float *v, int64_t ldv, int32_t max_rank, void *y, int64_t ldy,
                            int32_t d_out, bool ranks_vec, ExpandArgs *ea)
{
    int st = check_dtype(dtype);
    if (st) return st;
    if (!y) return fail(LORA_ERR_ARG, "y is NULL");
    if (d_out < 1) return fail(LORA_ERR_ARG, "d_out %d < 1", d_out);
    if (ldy < d_out) return fail(LORA_ERR_ARG, "ldy %lld < d_out %d", (long long)ldy, d_out);
    const int es = esize_of(dtype);
    if (!elem_aligned(y, es)) return fail(LORA_ERR_ALIGN, "y is not aligned to its element size");
    if ((st = check_v(v, ldv, max_rank))) return st;
    ea->dtype = dtype;
    ea->v = v;
    ea->ldv = ldv;
    ea->y = y;
    ea->ldy = ldy;
    ea->d_out = d_out;
    ea->vec_b = ranks_vec;
    ea->vec_y = aligned16(y) && ((ldy * es) % 16 == 0);
    return LORA_OK;
}

int bgmv_run(hipStream_t s, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in, const int32_t *ids_dev,
             const uint64_t *pool_A_dev, const uint64_t *pool_B_dev, const int32_t *pool_rank_dev,
             const float *pool_alpha_dev, int32_t n_adapters, int32_t max_rank, void *y, int64_t ldy, int32_t d_out,
             float *part, int32_t *ctl, bool one_launch)
{
    const int64_t ldw = (max_rank + 3) / 4 * 4;
    ShrinkArgs sa{};
    int st = make_shrink_args(dtype, x, ldx, d_in, part, ldw, max_rank, &sa);
    if (st) return st;
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, part, ldw, max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_bgmv(s, sa, ea, T, ids_dev, pool_A_dev, pool_B_dev, pool_rank_dev, pool_alpha_dev, n_adapters,
                       max_rank, part, ctl, one_launch);
}

} // namespace lora

using namespace lora;

extern "C" {

int lora_profile_launches(void **start_events, void **stop_events, int32_t count)
{
    clear_error();
    if (count < 0) return fail(LORA_ERR_ARG, "count %d < 0", count);
    if (count > 0 && (!start_events || !stop_events)) return fail(LORA_ERR_ARG, "event arrays are NULL");
    for (int32_t i = 0; i < count; ++i)
        if (!start_events[i] || !stop_events[i]) return fail(LORA_ERR_ARG, "event %d is NULL", i);
    LaunchEvents &le = launch_events();
    le.start = start_events;
    le.stop = stop_events;
    le.count = count;
    le.next = 0;
    return LORA_OK;
}

int32_t lora_profile_launches_used(void) { return launch_events().next; }

const char *lora_version(void) { return "lora_mi355x 0.1.0 (gfx950)"; }

const char *lora_last_error(void) { return g_last_error; }

const char *lora_status_string(int status)
{
    switch (status) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_ARG: return "LORA_ERR_ARG";
    case LORA_ERR_RANK: return "LORA_ERR_RANK";
    case LORA_ERR_ADAPTER_ID: return "LORA_ERR_ADAPTER_ID";
    case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN";
    case LORA_ERR_DTYPE: return "LORA_ERR_DTYPE";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
    case LORA_ERR_PLAN: return "LORA_ERR_PLAN";
    default: return "LORA_ERR_UNKNOWN";
    }
}

int64_t lora_adapter_numel(int32_t r, int32_t d_in, int32_t d_out)
{
    if (r < 0 || d_in < 0 || d_out < 0) return -1;
    return int64_t(r) * (int64_t(d_in) + int64_t(d_out));
}

size_t lora_segments_bytes(int32_t capacity)
{
    if (capacity < 0) capacity = 0;
    const size_t c = size_t(capacity);
    // header, segment descriptors (S <= T), block descriptors (blocks <= T'),
    // perm (T), chunk descriptors (chunks <= T'), segment index (T' <= T), the
    // segment arrays (S <= T), alignment slack
    return sizeof(lora_plan_header) + sizeof(lora_seg_desc) * c + 128 + sizeof(lora_blk_desc) * c + 4 * c + 64 +
           sizeof(lora_chunk_desc) * c + 4 * c + 16 + soa_bytes(capacity) + 16;
}

size_t lora_workspace_bytes(int op, int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank)
{
    (void)d_out;
    switch (op) {
    case LORA_OP_SGMV_SHRINK:
    case LORA_OP_SGMV_EXPAND:
    case LORA_OP_BGMV_SHRINK:
    case LORA_OP_BGMV_EXPAND: return 0;
    case LORA_OP_FUSED: return fused_workspace_bytes(T < 0 ? 0 : T, d_in < 1 ? 1 : d_in, max_rank < 1 ? 1 : max_rank);
    case LORA_OP_SGMV: // control words, fp32 partials (two kernels), tagged partials (one launch)
        return sgmv_ctl_bytes(T < 0 ? 0 : T) +
               3 * combined_workspace_bytes(T < 0 ? 0 : T, d_in < 1 ? 1 : d_in, max_rank < 1 ? 1 : max_rank);
    case LORA_OP_BGMV:
        return bgmv_workspace_bytes(T < 0 ? 0 : T, d_in < 1 ? 1 : d_in, max_rank < 1 ? 1 : max_rank);
    default: return size_t(-1);
    }
}

// The plan of one batch in `plan` (plan_bytes >= segments_bytes(T)): see the
// layout in the public header.  Pure host work, O(T + n_adapters).
static int build_plan(int32_t T, const int32_t *ids, int32_t n_adapters, const uint64_t *pool_A,
                      const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha, void *plan,
                      size_t plan_bytes)
{
    if (T < 0) return fail(LORA_ERR_ARG, "T %d < 0", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (!plan) return fail(LORA_ERR_ARG, "plan is NULL");
    if (reinterpret_cast<uintptr_t>(plan) & 15u) return fail(LORA_ERR_ALIGN, "buffer is not 16-byte aligned");
    if (plan_bytes < lora_segments_bytes(T))
        return fail(LORA_ERR_WORKSPACE, "buffer of %zu B < %zu B needed for %d tokens", plan_bytes,
                    lora_segments_bytes(T), T);
    if (T > 0 && !ids) return fail(LORA_ERR_ARG, "ids is NULL");

    // Count tokens per adapter; reject ids outside [-1, n_adapters).
    static thread_local std::vector<int32_t> count;
    count.assign(size_t(n_adapters), 0);
    int32_t sorted = 0;
    for (int32_t t = 0; t < T; ++t) {
        const int32_t a = ids[t];
        if (a < -1 || a >= n_adapters)
            return fail(LORA_ERR_ADAPTER_ID, "ids[%d] = %d outside [-1, %d)", t, a, n_adapters);
        if (a >= 0) {
            ++count[size_t(a)];
            ++sorted;
        }
    }
    if (sorted > 0 && (!pool_A || !pool_B || !pool_rank || !pool_alpha))
        return fail(LORA_ERR_ARG, "pool tables are NULL");

    // Segments in ascending adapter id; check the adapters actually used.
    int32_t S = 0, nblk = 0, nchunk = 0, max_rank = 0, max_len = 0;
    for (int32_t a = 0; a < n_adapters; ++a) {
        if (!count[size_t(a)]) continue;
        const int32_t r = pool_rank[a];
        if (r < 1 || r > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "adapter %d has rank %d outside [1, 256]", a, r);
        if (!pool_A[a] || !pool_B[a]) return fail(LORA_ERR_ARG, "adapter %d has a NULL A or B address", a);
        if ((pool_A[a] & 15u) || (pool_B[a] & 15u))
            return fail(LORA_ERR_ALIGN, "adapter %d: A or B address is not 16-byte aligned", a);
        ++S;
        const int32_t nb = (count[size_t(a)] + LORA_PLAN_ROW_BLOCK - 1) / LORA_PLAN_ROW_BLOCK;
        nblk += nb;
        nchunk += (nb + LORA_PLAN_CHUNK_BLOCKS - 1) / LORA_PLAN_CHUNK_BLOCKS;
        if (r > max_rank) max_rank = r;
        if (count[size_t(a)] > max_len) max_len = count[size_t(a)];
    }

    char *base = static_cast<char *>(plan);
    auto *h = reinterpret_cast<lora_plan_header *>(base);
    std::memset(h, 0, sizeof *h);
    h->num_tokens = T;
    h->num_sorted = sorted;
    h->num_segments = S;
    h->num_blocks = nblk;
    h->max_rank = max_rank;
    h->max_len = max_len;
    h->num_chunks = nchunk;
    h->seg_offset = sizeof(lora_plan_header);
    h->blk_offset = (h->seg_offset + sizeof(lora_seg_desc) * size_t(S) + 127) & ~size_t(127);
    h->perm_offset = align16(h->blk_offset + sizeof(lora_blk_desc) * size_t(nblk));
    h->chunk_offset = (h->perm_offset + 4 * size_t(T) + 63) & ~size_t(63);
    h->segidx_offset = align16(h->chunk_offset + sizeof(lora_chunk_desc) * size_t(nchunk));
    h->soa_offset = align16(h->segidx_offset + 4 * size_t(sorted));
    h->bytes_used = h->soa_offset + soa_bytes(S);

    auto *seg = reinterpret_cast<lora_seg_desc *>(base + h->seg_offset);
    auto *blk = reinterpret_cast<lora_blk_desc *>(base + h->blk_offset);
    auto *perm = reinterpret_cast<int32_t *>(base + h->perm_offset);
    auto *chunks = reinterpret_cast<lora_chunk_desc *>(base + h->chunk_offset);
    auto *segidx = reinterpret_cast<int32_t *>(base + h->segidx_offset);

    // Prefix offsets (reusing count as the running write position), descriptors
    // and the block list.
    int32_t s = 0, pos = 0, b = 0, ch = 0;
    for (int32_t a = 0; a < n_adapters; ++a) {
        const int32_t c = count[size_t(a)];
        if (!c) continue;
        lora_seg_desc &d = seg[s];
        d.A = pool_A[a];
        d.B = pool_B[a];
        d.start = pos;
        d.len = c;
        d.rank = pool_rank[a];
        d.adapter = a;
        d.scale = pool_alpha[a] / float(pool_rank[a]);
        d.blk0 = b;
        const int32_t nb = (c + LORA_PLAN_ROW_BLOCK - 1) / LORA_PLAN_ROW_BLOCK;
        for (int32_t i = 0; i < nb; i += LORA_PLAN_CHUNK_BLOCKS, ++ch) {
            lora_chunk_desc &k = chunks[ch];
            std::memset(&k, 0, sizeof k);
            k.A = d.A;
            k.B = d.B;
            k.scale = d.scale;
            k.rank = d.rank;
            k.p0 = pos + i * LORA_PLAN_ROW_BLOCK;
            k.n = std::min(LORA_PLAN_CHUNK_ROWS, c - i * LORA_PLAN_ROW_BLOCK);
            k.seg = s;
            k.first_blk = b + i;
            k.nblk = std::min(LORA_PLAN_CHUNK_BLOCKS, nb - i);
            for (int32_t m = 0; m < LORA_PLAN_CHUNK_ROWS; ++m) k.rows[m] = -1;
        }
        for (int32_t i = 0; i < nb; ++i, ++b) {
            lora_blk_desc &k = blk[b];
            std::memset(&k, 0, sizeof k);
            k.A = d.A;
            k.B = d.B;
            k.scale = d.scale;
            k.rank = d.rank;
            k.p0 = pos + i * LORA_PLAN_ROW_BLOCK;
            k.n = std::min(LORA_PLAN_ROW_BLOCK, c - i * LORA_PLAN_ROW_BLOCK);
            k.seg = s;
            for (int32_t m = 0; m < LORA_PLAN_ROW_BLOCK; ++m) k.rows[m] = -1;
        }
        count[size_t(a)] = pos;
        pos += c;
        ++s;
    }
    // Stable scatter: tokens in their original order; each lands in its
    // block's row list too (block of sorted position p is blk0 + (p - start) / 16).
    // Tokens without an adapter follow in their original order (perm[T' .. T)).
    for (int32_t t = 0, rest = sorted; t < T; ++t) {
        const int32_t a = ids[t];
        if (a < 0) {
            perm[rest++] = t;
            continue;
        }
        const int32_t p = count[size_t(a)]++;
        perm[p] = t;
    }
    for (int32_t si = 0, c0 = 0; si < S; ++si) {
        const lora_seg_desc &d = seg[si];
        for (int32_t q = 0; q < d.len; ++q) segidx[d.start + q] = si;
        for (int32_t q = 0; q < d.len; ++q) {
            blk[d.blk0 + q / LORA_PLAN_ROW_BLOCK].rows[q % LORA_PLAN_ROW_BLOCK] = perm[d.start + q];
            chunks[c0 + q / LORA_PLAN_CHUNK_ROWS].rows[q % LORA_PLAN_CHUNK_ROWS] = perm[d.start + q];
        }
        c0 += (d.len + LORA_PLAN_CHUNK_ROWS - 1) / LORA_PLAN_CHUNK_ROWS;
    }
    // the segment table as arrays (seg_A, seg_B, seg_indptr, seg_adapter,
    // seg_rank, seg_scale)
    SoA t = soa_at(base + h->soa_offset, S);
    for (int32_t si = 0; si < S; ++si) {
        t.A[si] = seg[si].A;
        t.B[si] = seg[si].B;
        t.indptr[si] = seg[si].start;
        t.adapter[si] = seg[si].adapter;
        t.rank[si] = seg[si].rank;
        t.scale[si] = seg[si].scale;
    }
    t.indptr[S] = sorted;
    h->magic = LORA_PLAN_MAGIC;
    return LORA_OK;
}

// Pointer and count fields of a segments struct bound to `buf` holding the plan.
static void fill_segments(lora_segments *s, char *buf, const lora_plan_header *h)
{
    const SoA t = soa_at(buf + h->soa_offset, h->num_segments);
    s->num_segments = h->num_segments;
    s->num_tokens = h->num_sorted;
    s->max_rank = h->max_rank;
    s->batch_tokens = h->num_tokens;
    s->perm = reinterpret_cast<int32_t *>(buf + h->perm_offset);
    s->seg_indptr = t.indptr;
    s->seg_adapter = t.adapter;
    s->seg_rank = t.rank;
    s->seg_A = t.A;
    s->seg_B = t.B;
    s->seg_scale = t.scale;
}

int lora_segments_bind(void *buf, int32_t capacity, lora_segments *out)
{
    clear_error();
    if (!out) return fail(LORA_ERR_ARG, "out is NULL");
    if (!buf) return fail(LORA_ERR_ARG, "buf is NULL");
    if (capacity < 0) return fail(LORA_ERR_ARG, "capacity %d < 0", capacity);
    if (!aligned16(buf)) return fail(LORA_ERR_ALIGN, "buf is not 16-byte aligned");
    std::memset(out, 0, sizeof *out);
    out->capacity = capacity;
    out->buf = buf;
    return LORA_OK;
}

int lora_build_segments(int32_t T, const int32_t *ids, int32_t n_adapters, const uint64_t *pool_A,
                        const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha,
                        lora_segments *out_host)
{
    clear_error();
    if (!out_host || !out_host->buf) return fail(LORA_ERR_ARG, "segments are not bound to a buffer");
    if (T > out_host->capacity)
        return fail(LORA_ERR_WORKSPACE, "batch of %d tokens > capacity %d", T, out_host->capacity);
    out_host->host = nullptr;
    const int st = build_plan(T, ids, n_adapters, pool_A, pool_B, pool_rank, pool_alpha, out_host->buf,
                              lora_segments_bytes(out_host->capacity));
    if (st) return st;
    char *buf = static_cast<char *>(out_host->buf);
    fill_segments(out_host, buf, reinterpret_cast<const lora_plan_header *>(buf));
    return LORA_OK;
}

int lora_segments_upload(const lora_segments *host, lora_segments *dev, void *stream)
{
    clear_error();
    if (!host || !dev) return fail(LORA_ERR_ARG, "host or dev is NULL");
    const lora_plan_header *h = nullptr;
    int st = check_plan(host->buf, &h);
    if (st) return st;
    if (!dev->buf) return fail(LORA_ERR_ARG, "dev is not bound to a buffer");
    if (dev->buf == host->buf) return fail(LORA_ERR_ARG, "dev and host are bound to the same buffer");
    if (lora_segments_bytes(dev->capacity) < h->bytes_used)
        return fail(LORA_ERR_WORKSPACE, "dev holds %d tokens; the batch has %d", dev->capacity, h->num_tokens);
    hipError_t e = hipMemcpyAsync(dev->buf, host->buf, h->bytes_used, hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
    fill_segments(dev, static_cast<char *>(dev->buf), h);
    dev->host = host->buf;
    return LORA_OK;
}

int lora_sgmv_shrink(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in, const lora_segments *seg,
                     float *v, int64_t ldv, void *ws, size_t ws_bytes)
{
    (void)ws;
    (void)ws_bytes;
    clear_error();
    const lora_plan_header *h = nullptr;
    const char *plan_dev = nullptr;
    int st = check_segments(seg, &h, &plan_dev);
    if (st) return st;
    if ((st = check_dtype(dtype))) return st;
    if (h->num_sorted == 0) return LORA_OK;
    if (!plan_dev) return fail(LORA_ERR_ARG, "the segments' device buffer is NULL");
    ShrinkArgs sa{};
    if ((st = make_shrink_args(dtype, x, ldx, d_in, v, ldv, h->max_rank, &sa))) return st;
    return launch_sgmv_shrink(static_cast<hipStream_t>(stream), sa, PlanView{h, plan_dev});
}

int lora_sgmv_expand(void *stream, int dtype, const float *v, int64_t ldv, const lora_segments *seg, void *y,
                     int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes)
{
    (void)ws;
    (void)ws_bytes;
    clear_error();
    const lora_plan_header *h = nullptr;
    const char *plan_dev = nullptr;
    int st = check_segments(seg, &h, &plan_dev);
    if (st) return st;
    if ((st = check_dtype(dtype))) return st;
    if (h->num_sorted == 0) return LORA_OK;
    if (!plan_dev) return fail(LORA_ERR_ARG, "the segments' device buffer is NULL");
    // B rows are r_s elements long: vector loads of 4 elements need r % 4 == 0 for
    // every segment; decided per segment on the device, so pass true here.
    if (h->num_blocks > 65535) return fail(LORA_ERR_ARG, "plan has %d blocks (> 65535)", h->num_blocks);
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, v, ldv, h->max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_sgmv_expand(static_cast<hipStream_t>(stream), ea, PlanView{h, plan_dev});
}

int lora_sgmv(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in, const lora_segments *seg, void *y,
              int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes)
{
    clear_error();
    const lora_plan_header *h = nullptr;
    const char *plan_dev = nullptr;
    int st = check_segments(seg, &h, &plan_dev);
    if (st) return st;
    if ((st = check_dtype(dtype))) return st;
    if (h->num_sorted == 0) return LORA_OK;
    if (!plan_dev) return fail(LORA_ERR_ARG, "the segments' device buffer is NULL");
    if (h->num_blocks > 65535) return fail(LORA_ERR_ARG, "plan has %d blocks (> 65535)", h->num_blocks);
    // the 256-byte status block, then the fp32 partials of the two-kernel
    // form, then the tagged 64-bit partials of the one-launch form
    const size_t ctl_bytes = sgmv_ctl_bytes(h->num_blocks);
    const size_t need = ctl_bytes + 3 * combined_workspace_bytes(h->num_sorted, d_in < 1 ? 1 : d_in, h->max_rank);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    const int64_t ldw = (h->max_rank + 3) / 4 * 4;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + ctl_bytes);
    ShrinkArgs sa{};
    if ((st = make_shrink_args(dtype, x, ldx, d_in, part, ldw, h->max_rank, &sa))) return st;
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, part, ldw, h->max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_sgmv(static_cast<hipStream_t>(stream), sa, ea, PlanView{h, plan_dev}, part,
                       static_cast<int32_t *>(ws));
}

int lora_bgmv(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in, const int32_t *ids_dev,
              const uint64_t *pool_A_dev, const uint64_t *pool_B_dev, const int32_t *pool_rank_dev,
              const float *pool_alpha_dev, int32_t n_adapters, int32_t max_rank, void *y, int64_t ldy, int32_t d_out,
              void *ws, size_t ws_bytes)
{
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "max_rank %d outside [1, 256]", max_rank);
    if (T == 0) return LORA_OK;
    if (!ids_dev || !pool_A_dev || !pool_B_dev || !pool_rank_dev || !pool_alpha_dev)
        return fail(LORA_ERR_ARG, "device tables are NULL");
    const size_t need = bgmv_workspace_bytes(T, d_in < 1 ? 1 : d_in, max_rank);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + bgmv_ctl_bytes(T));
    return bgmv_run(static_cast<hipStream_t>(stream), dtype, T, x, ldx, d_in, ids_dev, pool_A_dev, pool_B_dev,
                    pool_rank_dev, pool_alpha_dev, n_adapters, max_rank, y, ldy, d_out, part,
                    static_cast<int32_t *>(ws), true);
}

int lora_workspace_clear(void *stream, void *ws, size_t ws_bytes)
{
    clear_error();
    if (ws_bytes == 0) return LORA_OK;
    if (!ws) return fail(LORA_ERR_ARG, "ws is NULL");
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    return launch_workspace_clear(static_cast<hipStream_t>(stream), ws, ws_bytes);
}

int lora_debug_wait_limit(int32_t polls)
{
    clear_error();
    wait_limit() = polls;
    return LORA_OK;
}

// pages / page_bytes of the paged calls; *shift = log2(page_bytes).
static int check_pages(const void *pages, int64_t page_bytes, int *shift)
{
    if (!pages) return fail(LORA_ERR_ARG, "pages is NULL");
    if (!aligned16(pages)) return fail(LORA_ERR_ALIGN, "pages is not 16-byte aligned");
    if (lora_pages_needed(0, page_bytes) < 0)
        return fail(LORA_ERR_ARG, "page_bytes %lld is not a power of two in [64, 2^24]", (long long)page_bytes);
    int sh = 0;
    while ((int64_t(1) << sh) < page_bytes) ++sh;
    *shift = sh;
    return LORA_OK;
}

int lora_sgmv_paged(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in, const lora_segments *seg,
                    const void *pages, int64_t page_bytes, void *y, int64_t ldy, int32_t d_out, void *ws,
                    size_t ws_bytes)
{
    clear_error();
    const lora_plan_header *h = nullptr;
    const char *plan_dev = nullptr;
    int st = check_segments(seg, &h, &plan_dev);
    if (st) return st;
    if ((st = check_dtype(dtype))) return st;
    int shift = 0;
    if ((st = check_pages(pages, page_bytes, &shift))) return st;
    if (h->num_sorted == 0) return LORA_OK;
    if (!plan_dev) return fail(LORA_ERR_ARG, "the segments' device buffer is NULL");
    if (h->num_blocks > 65535) return fail(LORA_ERR_ARG, "plan has %d blocks (> 65535)", h->num_blocks);
    // the workspace of lora_sgmv (this call runs the two-kernel form and uses
    // its control words and fp32 partials)
    const size_t ctl_bytes = sgmv_ctl_bytes(h->num_blocks);
    const size_t need = ctl_bytes + 3 * combined_workspace_bytes(h->num_sorted, d_in < 1 ? 1 : d_in, h->max_rank);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    const int64_t ldw = (h->max_rank + 3) / 4 * 4;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + ctl_bytes);
    ShrinkArgs sa{};
    if ((st = make_shrink_args(dtype, x, ldx, d_in, part, ldw, h->max_rank, &sa))) return st;
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, part, ldw, h->max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_sgmv_paged(static_cast<hipStream_t>(stream), sa, ea, PlanView{h, plan_dev}, part, pages, shift);
}

int lora_bgmv_paged(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                    const int32_t *ids_dev, const uint64_t *pool_A_dev, const uint64_t *pool_B_dev,
                    const int32_t *pool_rank_dev, const float *pool_alpha_dev, int32_t n_adapters,
                    int32_t max_rank, const void *pages, int64_t page_bytes, void *y, int64_t ldy, int32_t d_out,
                    void *ws, size_t ws_bytes)
{
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    int shift = 0;
    if ((st = check_pages(pages, page_bytes, &shift))) return st;
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "max_rank %d outside [1, 256]", max_rank);
    if (T == 0) return LORA_OK;
    if (!ids_dev || !pool_A_dev || !pool_B_dev || !pool_rank_dev || !pool_alpha_dev)
        return fail(LORA_ERR_ARG, "device tables are NULL");
    const size_t need = bgmv_workspace_bytes(T, d_in < 1 ? 1 : d_in, max_rank);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    const int64_t ldw = (max_rank + 3) / 4 * 4;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + bgmv_ctl_bytes(T));
    ShrinkArgs sa{};
    if ((st = make_shrink_args(dtype, x, ldx, d_in, part, ldw, max_rank, &sa))) return st;
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, part, ldw, max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_bgmv_paged(static_cast<hipStream_t>(stream), sa, ea, T, ids_dev, pool_A_dev, pool_B_dev,
                             pool_rank_dev, pool_alpha_dev, n_adapters, max_rank, part, static_cast<int32_t *>(ws),
                             pages, shift);
}

size_t lora_sgmv_grouped_workspace_bytes(const lora_sgmv_proj *projs, int32_t n_proj)
{
    if (!projs || n_proj < 1 || n_proj > LORA_MAX_PROJ) return 0;
    size_t total = 0;
    for (int p = 0; p < n_proj; ++p) {
        const lora_plan_header *h = nullptr;
        const char *dev = nullptr;
        if (check_segments(projs[p].seg, &h, &dev)) return 0;
        clear_error();
        total += grouped_region_bytes(h->num_sorted, projs[p].d_in < 1 ? 1 : projs[p].d_in,
                                      h->max_rank < 1 ? 1 : h->max_rank);
    }
    return total;
}

int lora_sgmv_grouped(void *stream, int dtype, const lora_sgmv_proj *projs, int32_t n_proj, void *ws,
                      size_t ws_bytes)
{
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (!projs) return fail(LORA_ERR_ARG, "projs is NULL");
    if (n_proj < 1 || n_proj > LORA_MAX_PROJ)
        return fail(LORA_ERR_ARG, "n_proj %d outside [1, %d]", n_proj, LORA_MAX_PROJ);
    GroupedSgmv g[LORA_MAX_PROJ];
    size_t need = 0;
    for (int p = 0; p < n_proj; ++p) {
        const lora_sgmv_proj &q = projs[p];
        const lora_plan_header *h = nullptr;
        const char *plan_dev = nullptr;
        if ((st = check_segments(q.seg, &h, &plan_dev))) return st;
        for (int o = 0; o < p; ++o)
            if (projs[o].y == q.y) return fail(LORA_ERR_ARG, "projections %d and %d write the same y", o, p);
        g[p].plan = PlanView{h, plan_dev};
        g[p].ws = nullptr;
        if (h->num_sorted == 0) {
            g[p].sa = ShrinkArgs{};
            g[p].ea = ExpandArgs{};
            continue;
        }
        if (!plan_dev) return fail(LORA_ERR_ARG, "projection %d: the segments' device buffer is NULL", p);
        if (h->num_blocks > 65535) return fail(LORA_ERR_ARG, "projection %d: plan has %d blocks", p, h->num_blocks);
        need += grouped_region_bytes(h->num_sorted, q.d_in < 1 ? 1 : q.d_in, h->max_rank);
    }
    if (need == 0) return LORA_OK; // no projection has an adapted token
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    char *wp = static_cast<char *>(ws);
    for (int p = 0; p < n_proj; ++p) {
        const lora_sgmv_proj &q = projs[p];
        const lora_plan_header *h = g[p].plan.h;
        if (h->num_sorted == 0) continue;
        const int64_t ldw = (h->max_rank + 3) / 4 * 4;
        float *v = reinterpret_cast<float *>(wp);
        if ((st = make_shrink_args(dtype, q.x, q.ldx, q.d_in, v, ldw, h->max_rank, &g[p].sa)) ||
            (st = make_expand_args(dtype, v, ldw, h->max_rank, q.y, q.ldy, q.d_out, true, &g[p].ea))) {
            char msg[192];
            snprintf(msg, sizeof msg, "%s", lora_last_error()); // fail() rewrites the message buffer
            return fail(st, "projection %d: %s", p, msg);
        }
        g[p].ws = v;
        wp += grouped_region_bytes(h->num_sorted, q.d_in < 1 ? 1 : q.d_in, h->max_rank);
    }
    return launch_sgmv_grouped(static_cast<hipStream_t>(stream), g, n_proj);
}

size_t lora_bgmv_grouped_workspace_bytes(int32_t T, const lora_proj *projs, int32_t n_proj)
{
    if (T < 0 || !projs || n_proj < 1 || n_proj > LORA_MAX_PROJ) return 0;
    // the status block, then per projection: the two-launch form's fp32
    // partial sums and the one-launch form's tagged words (twice the bytes)
    size_t total = bgmv_ctl_bytes(T);
    for (int p = 0; p < n_proj; ++p) {
        const lora_proj &q = projs[p];
        if (q.max_rank < 1 || q.max_rank > LORA_MAX_RANK) return 0;
        total += 3 * grouped_region_bytes(T, q.d_in < 1 ? 1 : q.d_in, q.max_rank);
    }
    return total;
}

int lora_bgmv_grouped(void *stream, int dtype, int32_t T, const int32_t *ids_dev, int32_t n_adapters,
                      const lora_proj *projs, int32_t n_proj, void *ws, size_t ws_bytes)
{
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (!projs) return fail(LORA_ERR_ARG, "projs is NULL");
    if (n_proj < 1 || n_proj > LORA_MAX_PROJ)
        return fail(LORA_ERR_ARG, "n_proj %d outside [1, %d]", n_proj, LORA_MAX_PROJ);
    for (int p = 0; p < n_proj; ++p) {
        const lora_proj &q = projs[p];
        if (q.max_rank < 1 || q.max_rank > LORA_MAX_RANK)
            return fail(LORA_ERR_RANK, "projection %d: max_rank %d outside [1, 256]", p, q.max_rank);
        if (!q.pool_A_dev || !q.pool_B_dev || !q.pool_rank_dev || !q.pool_alpha_dev)
            return fail(LORA_ERR_ARG, "projection %d: device tables are NULL", p);
        for (int o = 0; o < p; ++o)
            if (projs[o].y == q.y) return fail(LORA_ERR_ARG, "projections %d and %d write the same y", o, p);
    }
    if (T == 0) return LORA_OK;
    if (!ids_dev) return fail(LORA_ERR_ARG, "ids_dev is NULL");
    const size_t need = lora_bgmv_grouped_workspace_bytes(T, projs, n_proj);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    GroupedProj gp[LORA_MAX_PROJ];
    int32_t *ctl = static_cast<int32_t *>(ws);
    char *region = static_cast<char *>(ws) + bgmv_ctl_bytes(T);
    for (int p = 0; p < n_proj; ++p) {
        const lora_proj &q = projs[p];
        const int64_t ldw = (q.max_rank + 3) / 4 * 4;
        float *v = reinterpret_cast<float *>(region);
        if ((st = make_shrink_args(dtype, q.x, q.ldx, q.d_in, v, ldw, q.max_rank, &gp[p].sa))) return st;
        if ((st = make_expand_args(dtype, v, ldw, q.max_rank, q.y, q.ldy, q.d_out, true, &gp[p].ea))) return st;
        gp[p].pool_A = q.pool_A_dev;
        gp[p].pool_B = q.pool_B_dev;
        gp[p].pool_rank = q.pool_rank_dev;
        gp[p].pool_alpha = q.pool_alpha_dev;
        gp[p].max_rank = q.max_rank;
        const size_t rb = grouped_region_bytes(T, q.d_in, q.max_rank);
        gp[p].part = reinterpret_cast<float *>(region + rb);
        region += 3 * rb;
    }
    return launch_bgmv_grouped(static_cast<hipStream_t>(stream), T, ids_dev, n_adapters, gp, n_proj, ctl);
}

int lora_bgmv_shrink(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                     const int32_t *ids_dev, const uint64_t *pool_A_dev, const int32_t *pool_rank_dev,
                     int32_t n_adapters, int32_t max_rank, float *v, int64_t ldv, void *ws, size_t ws_bytes)
{
    (void)ws;
    (void)ws_bytes;
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "max_rank %d outside [1, 256]", max_rank);
    if (T == 0) return LORA_OK;
    if (!ids_dev || !pool_A_dev || !pool_rank_dev) return fail(LORA_ERR_ARG, "device tables are NULL");
    ShrinkArgs sa{};
    if ((st = make_shrink_args(dtype, x, ldx, d_in, v, ldv, max_rank, &sa))) return st;
    return launch_bgmv_shrink(static_cast<hipStream_t>(stream), sa, T, ids_dev, pool_A_dev, pool_rank_dev,
                              n_adapters, max_rank);
}

int lora_bgmv_expand(void *stream, int dtype, int32_t T, const float *v, int64_t ldv, const int32_t *ids_dev,
                     const uint64_t *pool_B_dev, const int32_t *pool_rank_dev, const float *pool_alpha_dev,
                     int32_t n_adapters, int32_t max_rank, void *y, int64_t ldy, int32_t d_out, void *ws,
                     size_t ws_bytes)
{
    (void)ws;
    (void)ws_bytes;
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "max_rank %d outside [1, 256]", max_rank);
    if (T == 0) return LORA_OK;
    if (!ids_dev || !pool_B_dev || !pool_rank_dev || !pool_alpha_dev)
        return fail(LORA_ERR_ARG, "device tables are NULL");
    ExpandArgs ea{};
    if ((st = make_expand_args(dtype, v, ldv, max_rank, y, ldy, d_out, true, &ea))) return st;
    return launch_bgmv_expand(static_cast<hipStream_t>(stream), ea, T, ids_dev, pool_B_dev, pool_rank_dev,
                              pool_alpha_dev, n_adapters, max_rank);
}

// Checks and launch shared by the bf16 and E4M3 forms of the fused entry.
static int fused_common(void *stream, const void *x, int64_t ldx, int32_t d_in, const void *W0, int32_t d_out,
                        const lora_segments *seg, void *y, int64_t ldy, void *ws, size_t ws_bytes, bool e4m3,
                        float w0_scale)
{
    const lora_plan_header *h = nullptr;
    const char *plan_dev = nullptr;
    int st = check_segments(seg, &h, &plan_dev);
    if (st) return st;
    if (e4m3 && !(std::isfinite(w0_scale) && w0_scale != 0.0f))
        return fail(LORA_ERR_ARG, "w0_scale must be finite and non-zero");
    const int32_t T = h->num_tokens;
    if (T == 0) return LORA_OK;
    if (!x || !W0 || !y) return fail(LORA_ERR_ARG, "x, W0 or y is NULL");
    if (d_in < 1 || d_out < 1) return fail(LORA_ERR_ARG, "d_in %d or d_out %d < 1", d_in, d_out);
    if (ldx < d_in || ldy < d_out) return fail(LORA_ERR_ARG, "row pitch smaller than the row");
    if (!aligned16(x) || !aligned16(W0) || !aligned16(y) || (ldx * 2) % 16 || (ldy * 2) % 16 || (d_in * 2) % 16)
        return fail(LORA_ERR_ALIGN, "fused entry needs 16-byte aligned x, W0, y rows and d_in %% 8 == 0");
    if (e4m3 && d_in % 16)
        return fail(LORA_ERR_ALIGN, "an E4M3 W0 needs d_in %% 16 == 0 (16-byte rows), got %d", d_in);
    if (!plan_dev) return fail(LORA_ERR_ARG, "the segments' device buffer is NULL");
    const size_t need = fused_workspace_bytes(T, d_in, h->max_rank < 1 ? 1 : h->max_rank);
    if (!ws || ws_bytes < need) return fail(LORA_ERR_WORKSPACE, "workspace %zu B < %zu B needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(LORA_ERR_ALIGN, "workspace is not 16-byte aligned");
    ShrinkArgs sa{};
    sa.dtype = LORA_BF16;
    sa.x = x;
    sa.ldx = ldx;
    sa.d_in = d_in;
    sa.vec = true;
    ExpandArgs ea{};
    ea.dtype = LORA_BF16;
    ea.y = y;
    ea.ldy = ldy;
    ea.d_out = d_out;
    ea.vec_b = true;
    ea.vec_y = true;
    return launch_fused_linear(static_cast<hipStream_t>(stream), sa, W0, ea, PlanView{h, plan_dev}, ws, e4m3,
                               w0_scale);
}

int lora_fused_linear(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in, const void *W0,
                      int32_t d_out, const lora_segments *seg, void *y, int64_t ldy, void *ws, size_t ws_bytes)
{
    clear_error();
    int st = check_dtype(dtype);
    if (st) return st;
    if (dtype != LORA_BF16) return fail(LORA_ERR_DTYPE, "the fused entry takes bf16 only");
    return fused_common(stream, x, ldx, d_in, W0, d_out, seg, y, ldy, ws, ws_bytes, false, 1.0f);
}

int lora_fused_linear_e4m3(void *stream, const void *x, int64_t ldx, int32_t d_in, const void *W0, float w0_scale,
                           int32_t d_out, const lora_segments *seg, void *y, int64_t ldy, void *ws, size_t ws_bytes)
{
    clear_error();
    return fused_common(stream, x, ldx, d_in, W0, d_out, seg, y, ldy, ws, ws_bytes, true, w0_scale);
}

} // extern "C"

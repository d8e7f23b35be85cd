// Paged adapter storage: the frame allocator of a page pool and the kernel
// that writes a matrix into its frames.
//
// "Multi-LoRA Serving in Production ..." (llms.blog), section "Unified Paged
// Memory": adapter matrices are cut into fixed-size pages (16 KB or 64 KB are
// the sizes named there) held in non-contiguous frames of one HBM pool, with a
// software page table per matrix, so adapters are allocated and freed on
// demand without fragmenting memory.  The SGMV/BGMV kernels read paged
// matrices through their page tables (the PagedMem policy of the kernel file).
#include "internal.h"

#include <vector>

struct lora_page_alloc {
    std::vector<int32_t> free_stack; // top = back, taken next
    std::vector<uint8_t> taken;      // per frame
};

namespace lora {
namespace {

bool page_bytes_ok(int64_t page_bytes)
{
    return page_bytes >= 64 && page_bytes <= (int64_t(1) << 24) && (page_bytes & (page_bytes - 1)) == 0;
}

// Unit u (16 bytes, byte 16u of the matrix) goes to its page's frame.  A
// workgroup copies 1024 consecutive units, four per thread, all loads first.
// The last unit may be partial (bytes % 16): it is copied byte by byte so that
// nothing past the source is read.
__global__ __launch_bounds__(256) void pages_write_kernel(char *__restrict__ pages, int shift,
                                                          const int32_t *__restrict__ table,
                                                          const char *__restrict__ src, int64_t bytes)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int64_t full = bytes >> 4; // whole units
    const int64_t u0 = int64_t(blockIdx.x) * 1024 + threadIdx.x;
    const int64_t mask = (int64_t(1) << shift) - 1;
    u32x4 val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t u = u0 + 256 * i;
        if (u < full) val[i] = *reinterpret_cast<const u32x4 *>(src + 16 * u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t u = u0 + 256 * i;
        if (u < full) {
            const int64_t b = 16 * u;
            *reinterpret_cast<u32x4 *>(pages + ((int64_t(table[b >> shift]) << shift) | (b & mask))) = val[i];
        } else if (u == full && (bytes & 15)) {
            for (int64_t b = 16 * u; b < bytes; ++b) pages[(int64_t(table[b >> shift]) << shift) | (b & mask)] = src[b];
        }
    }
}

} // namespace
} // namespace lora

using namespace lora;

extern "C" {

int64_t lora_pages_needed(int64_t bytes, int64_t page_bytes)
{
    if (bytes < 0 || !page_bytes_ok(page_bytes)) return -1;
    return (bytes + page_bytes - 1) / page_bytes;
}

int lora_page_alloc_create(int32_t n_frames, lora_page_alloc **out)
{
    clear_error();
    if (!out) return fail(LORA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (n_frames < 1) return fail(LORA_ERR_ARG, "n_frames %d < 1", n_frames);
    auto *a = new lora_page_alloc;
    a->taken.assign(size_t(n_frames), 0);
    a->free_stack.resize(size_t(n_frames));
    // frame 0 on top: a fresh allocator hands out frames in ascending order
    for (int32_t f = 0; f < n_frames; ++f) a->free_stack[size_t(f)] = n_frames - 1 - f;
    *out = a;
    return LORA_OK;
}

void lora_page_alloc_destroy(lora_page_alloc *alloc) { delete alloc; }

int lora_page_alloc_take(lora_page_alloc *alloc, int32_t n, int32_t *frames_out)
{
    clear_error();
    if (!alloc) return fail(LORA_ERR_ARG, "alloc is NULL");
    if (n < 0) return fail(LORA_ERR_ARG, "n %d < 0", n);
    if (n == 0) return LORA_OK;
    if (!frames_out) return fail(LORA_ERR_ARG, "frames_out is NULL");
    if (size_t(n) > alloc->free_stack.size())
        return fail(LORA_ERR_WORKSPACE, "%d frames requested, %zu free", n, alloc->free_stack.size());
    for (int32_t i = 0; i < n; ++i) {
        const int32_t f = alloc->free_stack.back();
        alloc->free_stack.pop_back();
        alloc->taken[size_t(f)] = 1;
        frames_out[i] = f;
    }
    return LORA_OK;
}

int lora_page_alloc_give(lora_page_alloc *alloc, const int32_t *frames, int32_t n)
{
    clear_error();
    if (!alloc) return fail(LORA_ERR_ARG, "alloc is NULL");
    if (n < 0) return fail(LORA_ERR_ARG, "n %d < 0", n);
    if (n == 0) return LORA_OK;
    if (!frames) return fail(LORA_ERR_ARG, "frames is NULL");
    const size_t nf = alloc->taken.size();
    // validate everything first (2 = seen in this call), then commit
    int bad = -1;
    for (int32_t i = 0; i < n && bad < 0; ++i) {
        const int32_t f = frames[i];
        if (f < 0 || size_t(f) >= nf || alloc->taken[size_t(f)] != 1) bad = i;
        else alloc->taken[size_t(f)] = 2;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t f = frames[i];
        if (f >= 0 && size_t(f) < nf && alloc->taken[size_t(f)] == 2) alloc->taken[size_t(f)] = 1;
    }
    if (bad >= 0)
        return fail(LORA_ERR_ARG, "frame %d (entry %d) is out of range, not taken, or repeated", frames[bad], bad);
    for (int32_t i = 0; i < n; ++i) {
        alloc->taken[size_t(frames[i])] = 0;
        alloc->free_stack.push_back(frames[i]);
    }
    return LORA_OK;
}

int32_t lora_page_alloc_free_count(const lora_page_alloc *alloc)
{
    return alloc ? int32_t(alloc->free_stack.size()) : -1;
}

int lora_pages_write(void *stream, void *pages, int64_t page_bytes, const int32_t *table_dev, const void *src,
                     int64_t bytes)
{
    clear_error();
    if (!page_bytes_ok(page_bytes))
        return fail(LORA_ERR_ARG, "page_bytes %lld is not a power of two in [64, 2^24]", (long long)page_bytes);
    if (bytes < 0) return fail(LORA_ERR_ARG, "bytes %lld < 0", (long long)bytes);
    if (bytes == 0) return LORA_OK;
    if (!pages || !table_dev || !src) return fail(LORA_ERR_ARG, "pages, table_dev or src is NULL");
    if (!aligned16(pages) || !aligned16(src)) return fail(LORA_ERR_ALIGN, "pages or src is not 16-byte aligned");
    int shift = 0;
    while ((int64_t(1) << shift) < page_bytes) ++shift;
    const int64_t units = (bytes + 15) / 16;
    const int64_t blocks = (units + 1023) / 1024;
    if (blocks > 0x7fffffff) return fail(LORA_ERR_ARG, "bytes %lld too large", (long long)bytes);
    launch_kernel(pages_write_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                  static_cast<char *>(pages), shift, table_dev, static_cast<const char *>(src), bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "pages_write launch: %s", hipGetErrorString(e));
    return LORA_OK;
}

} // extern "C"

// Measurement aids: the "achievable at this size" references a benchmark
// reports beside the adapter kernels.
//
//  * probe_empty_kernel: a launch that does nothing (the per-launch floor);
//  * probe_stream_kernel: one launch that reads `read_bytes` of one buffer and
//    reads, modifies and writes back `rmw_bytes` of another, with 16-byte
//    accesses and four of them in flight per thread -- the same bytes an
//    adapter step must move (x, A and B read once, y read and written once)
//    with none of its dependent loads;
//  * probe_chase_kernel: one lane follows a chain of dependent loads (the
//    cost of one global-memory round trip inside a kernel).
#include "internal.h"

namespace lora {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4; // 16-byte accesses in flight per thread
constexpr int64_t kProbeTile = int64_t(kProbeThreads) * kProbeUnroll * 16; // bytes per workgroup step

__global__ __launch_bounds__(kProbeThreads) void probe_empty_kernel() {}

// Workgroups [0, rw) read their share of src; workgroups [rw, gridDim.x)
// read-modify-write their share of dst (x -> x ^ mask, mask = 0 at run time,
// so the data is unchanged but every store happens).  Byte counts are
// multiples of 16.
__global__ __launch_bounds__(kProbeThreads) void probe_stream_kernel(const u32x4 *__restrict__ src, int64_t n_read,
                                                                     u32x4 *__restrict__ dst, int64_t n_rmw, int rw,
                                                                     uint32_t mask, uint32_t *__restrict__ sink)
{
    const int b = int(blockIdx.x);
    if (b < rw) {
        u32x4 acc = u32x4{0, 0, 0, 0};
        const int64_t step = int64_t(rw) * kProbeThreads * kProbeUnroll;
        for (int64_t base = int64_t(b) * kProbeThreads * kProbeUnroll + threadIdx.x; base < n_read; base += step) {
            u32x4 v[kProbeUnroll];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) {
                const int64_t i = base + int64_t(u) * kProbeThreads;
                v[u] = src[i < n_read ? i : 0];
            }
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
        }
        // never true at run time (mask is 0); keeps the loads
        if (acc[0] == mask + 1u && acc[1] == 0x9e3779b9u) sink[b] = acc[2];
    } else {
        const int wb = b - rw, nw = int(gridDim.x) - rw;
        const int64_t step = int64_t(nw) * kProbeThreads * kProbeUnroll;
        for (int64_t base = int64_t(wb) * kProbeThreads * kProbeUnroll + threadIdx.x; base < n_rmw; base += step) {
            u32x4 v[kProbeUnroll];
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) {
                const int64_t i = base + int64_t(u) * kProbeThreads;
                v[u] = dst[i < n_rmw ? i : 0];
            }
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) {
                const int64_t i = base + int64_t(u) * kProbeThreads;
                if (i < n_rmw) dst[i] = v[u] ^ u32x4{mask, mask, mask, mask};
            }
        }
    }
}

// next[i] holds the index of the next element; `steps` dependent loads.
__global__ void probe_chase_kernel(const uint32_t *__restrict__ next, int steps, uint32_t *__restrict__ sink)
{
    uint32_t i = 0;
    for (int s = 0; s < steps; ++s) i = __builtin_nontemporal_load(next + i);
    if (threadIdx.x == 0) sink[0] = i;
}

// Workgroups for a part that moves `moved` of `total` bytes: its share of
// `total_wg`, at least one, at most one per kProbeTile of its `bytes`.
int grid_share(int64_t bytes, int64_t moved, int64_t total, int total_wg)
{
    if (bytes <= 0) return 0;
    const int64_t most = (bytes + kProbeTile - 1) / kProbeTile;
    int64_t share = (int64_t(total_wg) * moved + total - 1) / total;
    share = share < most ? share : most;
    return share < 1 ? 1 : int(share);
}

} // namespace
} // namespace lora

using namespace lora;

extern "C" {

int lora_probe_empty(void *stream, int32_t workgroups)
{
    clear_error();
    if (workgroups < 1) return fail(LORA_ERR_ARG, "workgroups %d < 1", workgroups);
    launch_kernel(probe_empty_kernel, dim3(unsigned(workgroups)), dim3(kProbeThreads), 0,
                  static_cast<hipStream_t>(stream));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? LORA_OK : fail(LORA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
}

int lora_probe_stream(void *stream, const void *src, int64_t read_bytes, void *rmw, int64_t rmw_bytes, void *sink,
                      int32_t max_workgroups)
{
    clear_error();
    if (read_bytes < 0 || rmw_bytes < 0 || (read_bytes | rmw_bytes) % 16)
        return fail(LORA_ERR_ARG, "byte counts must be non-negative multiples of 16");
    if ((read_bytes > 0 && !src) || (rmw_bytes > 0 && !rmw) || !sink) return fail(LORA_ERR_ARG, "NULL buffer");
    if (!aligned16(src) || !aligned16(rmw) || !aligned16(sink)) return fail(LORA_ERR_ALIGN, "buffers must be 16-byte aligned");
    if (max_workgroups < 2) return fail(LORA_ERR_ARG, "max_workgroups %d < 2", max_workgroups);
    if (read_bytes + rmw_bytes == 0) return LORA_OK;
    // workgroups split in proportion to the bytes each part moves (the RMW
    // part moves its bytes twice)
    const int64_t moved = read_bytes + 2 * rmw_bytes;
    const int rw = grid_share(read_bytes, read_bytes, moved, max_workgroups);
    const int wwr = grid_share(rmw_bytes, 2 * rmw_bytes, moved, max_workgroups);
    launch_kernel(probe_stream_kernel, dim3(unsigned(rw + wwr)), dim3(kProbeThreads), 0,
                  static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), read_bytes / 16,
                  static_cast<u32x4 *>(rmw), rmw_bytes / 16, rw, 0u, static_cast<uint32_t *>(sink));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? LORA_OK : fail(LORA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
}

int lora_probe_chase(void *stream, const uint32_t *next, int32_t steps, uint32_t *sink)
{
    clear_error();
    if (!next || !sink) return fail(LORA_ERR_ARG, "NULL buffer");
    if (steps < 0) return fail(LORA_ERR_ARG, "steps %d < 0", steps);
    launch_kernel(probe_chase_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), next, steps, sink);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? LORA_OK : fail(LORA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
}

} // extern "C"

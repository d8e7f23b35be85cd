// lora_bgmv_noalloc: the decode correction of lora_bgmv for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  It runs the shrink and expand
// kernels of lora_bgmv with their fp32 slice partials in a file-scope device
// array instead of a caller workspace.
//
// The array is one per device (each GPU the library runs on holds its own copy
// until the process ends).  Host code never uses its name as an address: on
// the first call on a device, with that device current, its device address is
// looked up once and kept per device.  The shrink writes every partial the
// expand reads before the expand runs, so nothing in the array has to start
// at any value and calls need no clearing.  Every call on one device shares
// the array: calls that overlap on one device (different streams without an
// ordering between them) race.
#include "internal.h"

#include <mutex>

namespace lora {
namespace {

constexpr size_t kScratchBytes = size_t(LORA_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of this device's scratch, looked up on first use.
int scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LORA_ERR_ARG, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail(LORA_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return LORA_OK;
}

} // namespace
} // namespace lora

using namespace lora;

extern "C" int lora_bgmv_noalloc(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                                 const int32_t *ids_dev, const uint64_t *pool_A_dev, const uint64_t *pool_B_dev,
                                 const int32_t *pool_rank_dev, const float *pool_alpha_dev, int32_t n_adapters,
                                 int32_t max_rank, void *y, int64_t ldy, int32_t d_out)
{
    clear_error();
    if (dtype != LORA_F32 && dtype != LORA_BF16) return fail(LORA_ERR_DTYPE, "unknown dtype %d", dtype);
    if (T < 0 || T > 65536) return fail(LORA_ERR_ARG, "T %d outside [0, 65536]", T);
    if (n_adapters < 0) return fail(LORA_ERR_ARG, "n_adapters %d < 0", n_adapters);
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return fail(LORA_ERR_RANK, "max_rank %d outside [1, 256]", max_rank);
    if (T == 0) return LORA_OK;
    if (!ids_dev || !pool_A_dev || !pool_B_dev || !pool_rank_dev || !pool_alpha_dev)
        return fail(LORA_ERR_ARG, "device tables are NULL");
    const size_t need = combined_workspace_bytes(T, d_in < 1 ? 1 : d_in, max_rank);
    if (need > kScratchBytes)
        return fail(LORA_ERR_WORKSPACE, "batch needs %zu B of partial sums; the static scratch holds %zu B", need,
                    kScratchBytes);
    void *part = nullptr;
    const int st = scratch_ptr(&part);
    if (st) return st;
    return bgmv_run(static_cast<hipStream_t>(stream), dtype, T, x, ldx, d_in, ids_dev, pool_A_dev, pool_B_dev,
                    pool_rank_dev, pool_alpha_dev, n_adapters, max_rank, y, ldy, d_out, static_cast<float *>(part),
                    nullptr, false);
}

// Internal declarations shared by the host shim and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "lora_mi355x.h"

namespace lora {

// Records the message of a failed call for lora_last_error() and returns status.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Parsed view of a plan: host header plus the device base address.
struct PlanView {
    const lora_plan_header *h; // host copy (counts, offsets)
    const char *dev;           // device copy (same layout)
};

// Launch geometry / path choices made on the host.
struct ShrinkArgs {
    int dtype;
    const void *x;
    int64_t ldx;
    int32_t d_in;
    float *v;
    int64_t ldv;
    bool vec; // 16-byte loads of x rows and A rows are legal
};

struct ExpandArgs {
    int dtype;
    const float *v;
    int64_t ldv;
    void *y;
    int64_t ldy;
    int32_t d_out;
    bool vec_b; // 8-byte (bf16) / 16-byte (f32) loads of B rows are legal
    bool vec_y; // 16-byte loads/stores of y rows are legal
};

int launch_sgmv_shrink(hipStream_t s, const ShrinkArgs &a, const PlanView &p);
int launch_sgmv_expand(hipStream_t s, const ExpandArgs &a, const PlanView &p);
int launch_bgmv_shrink(hipStream_t s, const ShrinkArgs &a, int32_t T, const int32_t *ids,
                       const uint64_t *pool_A, const int32_t *pool_rank, int32_t n_adapters,
                       int32_t max_rank);
int launch_bgmv_expand(hipStream_t s, const ExpandArgs &a, int32_t T, const int32_t *ids,
                       const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha,
                       int32_t n_adapters, int32_t max_rank);
// The combined SGMV: one launch over the plan's chunks (shrink and expand
// items handing over through tagged partial sums, with the sticky status word
// at `ctl`) when ctl is given and the shapes allow it, else the shrink and
// expand kernels.
int launch_sgmv(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, const PlanView &p, void *ws,
                int32_t *ctl = nullptr);
// Control words of an SGMV workspace for a plan of up to n_blocks blocks:
// the 256-byte status block.
size_t sgmv_ctl_bytes(int32_t n_blocks);
// The combined BGMV: one launch (shrink and expand workgroups in one grid,
// handing over through tagged partial sums after the slice partials, with
// the sticky status word at `ctl`) when one_launch and the shapes allow it,
// else the shrink and expand kernels.  ws: the slice partials.
int launch_bgmv(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank, const float *pool_alpha,
                int32_t n_adapters, int32_t max_rank, void *ws, int32_t *ctl, bool one_launch);
// A BGMV workspace: the 256-byte status block, the two-launch form's slice
// partials, then the one-launch form's tagged words (twice those bytes).
size_t bgmv_ctl_bytes(int32_t T);
size_t bgmv_workspace_bytes(int32_t T, int32_t d_in, int32_t max_rank);
// Argument checks of x, y and the partials, then launch_bgmv.  part: the slice
// partials; ctl: control words of the one-launch form (nullptr: two kernels).
int bgmv_run(hipStream_t s, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in, const int32_t *ids_dev,
             const uint64_t *pool_A_dev, const uint64_t *pool_B_dev, const int32_t *pool_rank_dev,
             const float *pool_alpha_dev, int32_t n_adapters, int32_t max_rank, void *y, int64_t ldy, int32_t d_out,
             float *part, int32_t *ctl, bool one_launch);
// Zero `bytes` of device memory with a kernel (no memset node in a graph).
int launch_workspace_clear(hipStream_t s, void *ws, size_t bytes);
// Polls of the one-launch BGMV's wait before it gives up (per thread; 0 = the
// default, < 0 = give up at once).
int &wait_limit();
// The combined SGMV / BGMV calls over paged adapter storage: the adapter
// table entries (plan descriptors, pool_A / pool_B) are int32 page tables of
// frames in `pages`, pages of 2^page_shift bytes.
int launch_sgmv_paged(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, const PlanView &p, void *ws,
                      const void *pages, int page_shift);
int launch_bgmv_paged(hipStream_t s, const ShrinkArgs &sa, const ExpandArgs &ea, int32_t T, const int32_t *ids,
                      const uint64_t *pool_A, const uint64_t *pool_B, const int32_t *pool_rank,
                      const float *pool_alpha, int32_t n_adapters, int32_t max_rank, void *ws, int32_t *ctl,
                      const void *pages, int page_shift);
// One projection of a grouped BGMV call: its shrink (x, d_in, v = its
// workspace region) and expand (y, d_out) arguments and its adapter tables.
struct GroupedProj {
    ShrinkArgs sa;
    ExpandArgs ea;
    const uint64_t *pool_A;
    const uint64_t *pool_B;
    const int32_t *pool_rank;
    const float *pool_alpha;
    float *part; // the one-launch form's tagged partial sums (a region of their own)
    int32_t max_rank;
};
// ctl: the workspace's status block (one launch when every projection fits
// it), or null for the two-launch form.
int launch_bgmv_grouped(hipStream_t s, int32_t T, const int32_t *ids, int32_t n_adapters, const GroupedProj *pr,
                        int n, int32_t *ctl);
// One projection of a grouped SGMV call: its plan, shrink and expand
// arguments, and its workspace region (the fp32 slice partials of v).
struct GroupedSgmv {
    ShrinkArgs sa;
    ExpandArgs ea;
    PlanView plan;
    float *ws;
};
int launch_sgmv_grouped(hipStream_t s, const GroupedSgmv *pr, int n);
// Bytes of one projection's region in a grouped workspace (256-byte multiple).
size_t grouped_region_bytes(int32_t T, int32_t d_in, int32_t max_rank);

// Workspace of the combined calls and of the fused entry: fp32 partial sums of
// the shrink over d_in slices.
size_t combined_workspace_bytes(int32_t rows, int32_t d_in, int32_t max_rank);
// SGMV shrink of every plan row into slice partials: ws[c * sl_stride + p * ldw + j]
// for slice c < *nsl, sorted position p, rank j < r (ranks r .. ldw-1 are not
// written).  ldw = round4(max_rank), sl_stride = T' * ldw.
int launch_sgmv_shrink_split(hipStream_t s, const ShrinkArgs &sa, const PlanView &p, float *ws, int64_t *ldw,
                             int64_t *sl_stride, int *nsl);
// w0_e4m3: W0 holds OCP E4M3 codes standing for w0_scale * code (finite,
// non-zero scale); otherwise bf16.
int launch_fused_linear(hipStream_t s, const ShrinkArgs &sa, const void *W0, const ExpandArgs &ea,
                        const PlanView &p, void *ws, bool w0_e4m3 = false, float w0_scale = 1.0f);
size_t fused_workspace_bytes(int32_t T, int32_t d_in, int32_t max_rank);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-thread request to time the next launches (lora_profile_launches).
struct LaunchEvents {
    void **start = nullptr;
    void **stop = nullptr;
    int count = 0;
    int next = 0;
};
LaunchEvents &launch_events();

// Every kernel launch of the library goes through here, so a pending timing
// request attaches its events to the kernel's own start and end.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    LaunchEvents &le = launch_events();
    if (le.next < le.count) {
        e0 = static_cast<hipEvent_t>(le.start[le.next]);
        e1 = static_cast<hipEvent_t>(le.stop[le.next]);
        ++le.next;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(shm), s, e0, e1, 0, static_cast<KArgs>(args)...);
}

} // namespace lora

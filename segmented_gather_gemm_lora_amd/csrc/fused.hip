// Fused adapted layer: y = x W0 + scale_s (x A_s) B_s (see lora_fused_linear).
#include "internal.h"

namespace lora {

size_t fused_workspace_bytes(int32_t T, int32_t max_rank)
{
    const size_t ldv = size_t((max_rank + 15) / 16 * 16);
    return size_t(T) * ldv * sizeof(float) + 256;
}

int launch_fused_linear(hipStream_t, const ShrinkArgs &, const void *, const ExpandArgs &, const PlanView &, void *,
                        size_t)
{
    return fail(LORA_ERR_ARG, "lora_fused_linear: not built in this version");
}

} // namespace lora

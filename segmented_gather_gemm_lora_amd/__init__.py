"""Multi-LoRA batched adapter path for AMD MI355X (gfx950).

y[t] += (alpha_i / r_i) * (x[t] A_i) B_i for every token t, adapter i = ids[t],
adapters resident in device memory with unpadded heterogeneous ranks.  The
work runs in hand-written HIP kernels behind a C ABI (include/lora_mi355x.h);
this package is the thin Python binding over it (see ``binding``).
"""

from .binding import (  # noqa: F401
    DTYPES,
    LORA_BF16,
    LORA_F32,
    DevicePool,
    LoraError,
    Plan,
    bgmv,
    bgmv_expand,
    bgmv_shrink,
    fused_linear,
    lib_path,
    load,
    sgmv,
    sgmv_expand,
    sgmv_shrink,
    to_device,
    to_host_bits,
    v_pitch,
    workspace,
)

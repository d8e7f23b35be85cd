"""Seeded synthetic inputs for the multi-LoRA batched adapter path.

This package is the only code that both the GPU path's tests/bench and the
CPU oracle's tests consume.  It draws random numbers and lays them out in
memory; it contains none of the method's arithmetic (no shrink, no expand, no
sort, no scale).  Every array is a numpy array on the host.
"""

from .synth import (  # noqa: F401
    LoraProblem,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_problem,
    make_integer_problem,
    make_decode_qkv,
    make_prefill_qkv,
    PREFILL_QKV_NAME,
    make_decode_registry,
    CACHE_NAME,
    QKV_NAME,
    CONFIG_NAMES,
    zipf_probs,
    e4m3_codes,
    with_e4m3_base,
    make_fused_fp8,
    FUSED_FP8_NAME,
)

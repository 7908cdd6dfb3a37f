"""Seeded synthetic workloads for FP8 MLA context prefill.

This package is the only code shared by the CPU oracle side and the GPU side.
It holds random draws and their rounding to bf16 input bytes, nothing of the
method itself: no FP8 encoding, no scales, no attention, no merge.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    D_QK,
    D_V,
    N_HEADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_codes,
    make_latent,
    make_workload,
    random_varlen,
)

"""FP8 MLA context prefill (Q/K head dim 192, V head dim 128) for MI355X (gfx950).

The compute lives in ``libmla_fp8.so`` (hand-written HIP kernels behind a C
ABI, ``include/mla_fp8.h``); ``binding`` is its thin ctypes binding.
"""

__all__ = ["binding", "build"]

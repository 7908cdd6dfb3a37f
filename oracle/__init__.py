"""CPU fp64 oracle for FP8 MLA context prefill. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from this package. The library and its Python
binding never import it, and this package never imports them: the two sides
share only the seeded input generators in ``synth``.

What it computes, and the passages it follows (all from the vLLM PR
"[ROCm][MLA] Add guarded gfx942 FP8 context prefill", #51551, unless noted):

  e4m3.py      OCP E4M3FN codec: decode table and saturating round-to-nearest-even
               encode (FP8 maximum = the dtype's finite maximum, as in the vLLM PR
               "[ROCm][Kimi-K3] Fuse gated RMSNorm with per-token FP8 for KDA o_proj",
               #54254, review thread on ``rmsnorm_gated_fp8_per_token``).
  quant.py     static per-head quantization with caller-supplied descales (Summary;
               "What this PR does": one-kernel static quantizer, finite positive
               descales), the calibration arithmetic descale = amax / 448, and the
               dynamic variant that takes the amax of the data itself (the per-head
               reduction the static path removes, Summary).
  attention.py softmax attention over packed variable-length sequences on the
               dequantized FP8 inputs, returning out and LSE (Background: packed
               variable-length D192/V128 kernel; "What this PR does": 12 heads,
               D192 Q/K, D128 V); the same definition on bf16 inputs is the BF16
               comparator of the close comment.
  merge.py     log-sum-exp merge of per-segment partials ("What this PR does": Q is
               quantized once and reused across context segments).
  chunked.py   segmented drivers: each context segment is attended separately and
               the partials merged; must equal the unsegmented result.
  producer.py  the un-absorbed MLA keys and values expanded from the latent cache per
               head (bf16 projection, rope part shared by the heads), then quantized
               (vLLM #60110, Purpose: prefill keeps the un-absorbed form; its
               shapes).

Parity pins: every function is checked by tests under ``tests/test_oracle_*.py``
against closed forms, exhaustive exact-rational rounding, brute force on tiny
inputs and invariants. The pages print no numeric example, so no pin comes from
the pages' own values.
"""

from .e4m3 import decode_table, e4m3_decode, e4m3_encode  # noqa: F401
from .quant import amax_per_head, descale_from_amax, quant_dynamic, quant_static  # noqa: F401
from .attention import (attention_rows, attention_rows_bf16, attention_varlen,  # noqa: F401
                        attention_varlen_bf16)
from .merge import merge_lse  # noqa: F401
from .chunked import chunked_context, segment_plan  # noqa: F401
from .producer import kv_produce, kv_project_bf16, rn_bf16_bits  # noqa: F401

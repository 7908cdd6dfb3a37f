"""Static per-head FP8 quantization and its calibration arithmetic.  (Oracle only.)

Follows the vLLM PR "[ROCm][MLA] Add guarded gfx942 FP8 context prefill"
(#51551): per-head static scales come from layer maxima collected in a
calibration pass and are loaded as finite positive descales (section "What
this PR does"); a one-kernel static quantizer then maps bf16 activations to
FP8 with no runtime amax reduction (Summary).

Readings (the pages give no formula):
  * descale[h] = RN_fp32(amax[h] / 448), amax = max |x| over all tokens and dims
    of head h in the calibration draw;
  * code = e4m3_encode(x / descale[h]): the correctly rounded E4M3 value of the
    exact quotient.

Why float64 division gives the correctly rounded result: x is bf16 (8
significant bits), descale is fp32 (24 bits) and an E4M3 rounding boundary M
has at most 5 significant bits. If x != M * descale, the two differ by at
least 2^-29 of their size, while the float64 quotient is off by at most 2^-53
relative. So the float64 quotient never lands on or across a boundary that the
exact quotient does not sit on, and it is exact when the quotient is a
boundary.

Why the descale is correctly rounded: amax has 8 significant bits and
448 = 7 * 2^6, so amax / 448 is either exact or a repeating binary fraction
with period 3; it is never within 2^-53 of an fp32 rounding boundary, so
rounding the float64 quotient to fp32 equals rounding the exact quotient.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quant_static(x_bits: np.ndarray, descale: np.ndarray) -> np.ndarray:
    """x_bits: uint16 bf16 patterns [T, H, D]; descale: float32 [H]. Returns uint8 codes [T, H, D]."""
    x = _bf16_to_f64(x_bits)
    d = np.asarray(descale, dtype=np.float32).astype(np.float64)
    if x.ndim != 3 or d.shape != (x.shape[1],):
        raise ValueError("x must be [T, H, D] and descale [H]")
    if not (np.all(np.isfinite(d)) and np.all(d > 0)):
        raise ValueError("descales must be finite and positive")
    return e4m3_encode(x / d[None, :, None])


def amax_per_head(x_bits: np.ndarray) -> np.ndarray:
    """Max |x| per head over tokens and dims, as float32 [H] (exact: bf16 values widen exactly)."""
    x = np.abs(_bf16_to_f64(x_bits))
    if x.shape[0] == 0:
        return np.zeros(x.shape[1], dtype=np.float32)
    return x.max(axis=(0, 2)).astype(np.float32)


def descale_from_amax(amax: np.ndarray) -> np.ndarray:
    """descale = RN_fp32(amax / 448); rejects amax that is not finite and positive."""
    a = np.asarray(amax, dtype=np.float32)
    if not (np.all(np.isfinite(a)) and np.all(a > 0)):
        raise ValueError("amax must be finite and positive")
    return (a.astype(np.float64) / E4M3_MAX).astype(np.float32)


FP32_MIN_NORMAL = 2.0 ** -126


def quant_dynamic(x_bits: np.ndarray):
    """Dynamic per-head quantization, the baseline the static path replaces (vLLM PR #51551,
    Summary: the static scales remove a per-head amax reduction from every prefill step).

    The amax is taken over the data being quantized: amax[h] = max |x| over its tokens and
    dims; descale[h] = RN_fp32(amax[h] / 448), floored at 2^-126 (the smallest normal fp32,
    so that 1/descale stays finite), or 1 for a head whose values are all zero (any positive
    descale gives the same codes there). Inputs must be finite. Returns (codes, descale)."""
    amax = amax_per_head(x_bits)
    if not np.all(np.isfinite(amax)):
        raise ValueError("dynamic quantization needs finite inputs")
    d = np.ones(amax.shape, dtype=np.float32)
    pos = amax > 0
    d[pos] = (amax[pos].astype(np.float64) / E4M3_MAX).astype(np.float32)
    d = np.maximum(d, np.float32(FP32_MIN_NORMAL)).astype(np.float32)
    return quant_static(x_bits, d), d

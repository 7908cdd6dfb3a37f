"""Descale sets for exhaustive quantizer tests (used by the oracle pins and the GPU parity).

``adversarial_descales`` searches, with a fixed seed, for fp32 descales d for
which the fp32-rounded quotient fl32(x / d) of some bf16 value x lands exactly
on an E4M3 rounding boundary although the exact quotient does not: the
double-rounding trap for a kernel that divides in fp32 and then rounds.
"""

from __future__ import annotations

import functools

import numpy as np

from tests.exact_e4m3 import MAGS


def all_bf16_patterns() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _bf16_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@functools.lru_cache(maxsize=None)
def adversarial_descales(count: int = 8, seed: int = 123) -> tuple:
    mids = np.array([float((MAGS[i] + MAGS[i + 1]) / 2) for i in range(126)], dtype=np.float64)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # midpoints are exact in fp32
    bits = all_bf16_patterns()
    x32 = _bf16_f32(bits)
    ok = np.isfinite(x32) & (x32 != 0)
    x32 = np.abs(x32[ok])
    x64 = x32.astype(np.float64)
    rng = np.random.default_rng(seed)
    found = []
    tries = 0
    while len(found) < count and tries < 20000:
        tries += 1
        d = np.float32(np.exp2(rng.uniform(-9.0, 3.0)))
        with np.errstate(over="ignore"):
            q32 = x32 / d  # fp32 quotient, correctly rounded
        hit = np.isin(q32, mids32)
        if not hit.any():
            continue
        # exact check: x == M * d exactly? (M * d is exact in float64: 5 + 24 bits)
        prod = q32[hit].astype(np.float64) * np.float64(d)
        if np.any(prod != x64[hit]):
            found.append(float(d))
    return tuple(found)


def standard_descales() -> tuple:
    return (1.0, 2.0 ** -3, 2.0 ** 5, 1.0 / 448.0, 3.0, 0.7, 4.0 / 448.0, 0.0123)

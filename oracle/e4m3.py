"""OCP E4M3FN codec, exact, in float64.  (Oracle: test infrastructure only.)

Format (OCP 8-bit floating point, E4M3 "fn" variant; named float8_e4m3fn on
MI355X in the vLLM PR "[ROCm][Perf] FP8 o-projection for DeepSeek-V4.1-Flash MLA
on AMD MI355X", #57081, section Purpose; saturation bound = the dtype's finite
maximum, 448, as in the vLLM PR "[ROCm][Kimi-K3] Fuse gated RMSNorm with
per-token FP8 for KDA o_proj", #54254, review thread on
rmsnorm_gated_fp8_per_token):

  code = s eeee mmm;  e = 0: (-1)^s * m * 2^-9 (subnormal)
                      e > 0: (-1)^s * (1 + m/8) * 2^(e-7)
                      e = 15, m = 7: NaN (no infinities)

Encoding of a real t (the reading used throughout; the pages do not spell out
the rounding rule):
  * NaN -> 0x7F with t's sign bit;
  * |t| > 448 (including infinities) -> 0x7E with t's sign (saturate);
  * otherwise the nearest of the 127 non-negative finite magnitudes, ties to
    the even code (even mantissa); the sign bit of t is kept, so -0 and
    negative values that round to zero give 0x80.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """float64[256]: value of every code; NaN for 0x7F and 0xFF."""
    c = np.arange(256, dtype=np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_TABLE = decode_table()
# non-negative finite magnitudes, codes 0x00..0x7E, strictly increasing
_MAGS = _TABLE[:127].copy()
# rounding boundaries between consecutive magnitudes (exact in float64)
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """Encode float64 values to uint8 codes: saturating, round to nearest, ties to even."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    # number of boundaries strictly below a = index of the lower neighbour, or the
    # nearest magnitude when a is not exactly on a boundary
    i = np.searchsorted(_MIDS, a, side="left")
    on_mid = np.zeros(a.shape, dtype=bool)
    inside = i < _MIDS.shape[0]
    on_mid[inside] = a[inside] == _MIDS[i[inside]]
    # a boundary between codes i and i+1: choose the even code
    i = np.where(on_mid & (i % 2 == 1), i + 1, i)
    # searchsorted already puts every a > 432 (and +inf) at i = 126 (0x7E): saturation
    code = i.astype(np.uint8)
    code = np.where(np.isnan(t), np.uint8(0x7F), code)
    sign = np.signbit(t).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)

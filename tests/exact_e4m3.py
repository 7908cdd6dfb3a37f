"""Independent exact-rational E4M3FN rounder used to pin the oracle and the kernels.

Written from the OCP E4M3FN definition with ``fractions.Fraction`` only: it
shares nothing with ``oracle/e4m3.py`` (which uses a float64 table and
``searchsorted``) or with the HIP quantizer (integer/fp32 bit manipulation).
"""

from __future__ import annotations

import bisect
from fractions import Fraction

# the 127 non-negative finite magnitudes, code order 0x00..0x7E
MAGS = [Fraction(m, 512) for m in range(8)] + [
    Fraction(8 + m, 8) * Fraction(2) ** (e - 7) for e in range(1, 16) for m in range(8)
][: 127 - 8]
assert len(MAGS) == 127 and MAGS[-1] == 448 and MAGS[8] == Fraction(1, 64)


def round_e4m3(q: Fraction, negative: bool) -> int:
    """Code of the correctly rounded, saturating E4M3FN value of the real number q."""
    a = abs(q)
    sign = 0x80 if negative else 0
    if a > 448:
        return 0x7E | sign
    i = bisect.bisect_left(MAGS, a)  # MAGS[i-1] < a <= MAGS[i]
    if i < 127 and MAGS[i] == a:
        return i | sign
    lo, hi = i - 1, i
    dlo, dhi = a - MAGS[lo], MAGS[hi] - a
    if dlo < dhi:
        c = lo
    elif dhi < dlo:
        c = hi
    else:
        c = lo if lo % 2 == 0 else hi
    return c | sign


def bf16_fraction(bits: int):
    """(Fraction value, negative flag, kind) for a bf16 pattern; kind in {'num','inf','nan'}."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return None, bool(s), ("nan" if m else "inf")
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** -126
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return v, bool(s), "num"


def f32_fraction(x) -> Fraction:
    return Fraction(float(x))


def quant_exact(bits: int, descale) -> int:
    """Expected code for bf16 pattern ``bits`` divided by fp32 ``descale`` (exact)."""
    v, neg, kind = bf16_fraction(bits)
    if kind == "nan":
        return 0x7F | (0x80 if neg else 0)
    if kind == "inf":
        return 0x7E | (0x80 if neg else 0)
    return round_e4m3(v / f32_fraction(descale), neg)


def round_fp32(q: Fraction) -> float:
    """Correctly rounded (ties to even) fp32 value of a positive rational in the normal range."""
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # find e with 2^e <= q < 2^(e+1)
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    assert -126 <= e <= 127
    scaled = q / Fraction(2) ** (e - 23)  # in [2^23, 2^24)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(Fraction(n) * Fraction(2) ** (e - 23))

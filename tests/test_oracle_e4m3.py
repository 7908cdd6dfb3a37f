"""Pins for the oracle's E4M3FN codec (oracle/e4m3.py).

Pinned against: values fixed by the OCP E4M3FN definition (hand-derived
spot values), torch's own float8_e4m3fn decoding on the CPU (an independent
library routine), an exact-rational rounder (tests/exact_e4m3.py), and the
round trip.
"""

import math

import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_encode, decode_table
from tests.exact_e4m3 import MAGS, round_e4m3
from fractions import Fraction


def test_spot_values_from_definition():
    t = decode_table()
    assert t[0x00] == 0.0 and not math.copysign(1.0, t[0x00]) < 0
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) < 0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x40] == 2.0
    assert t[0x3C] == 1.5
    assert t[0x7E] == 448.0              # largest finite
    assert t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    finite = t[:127]
    assert np.all(np.diff(finite) > 0)   # strictly increasing magnitudes


def test_decode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_decode_matches_exact_magnitudes():
    t = decode_table()
    for c in range(127):
        assert Fraction(t[c]) == MAGS[c]


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_specials():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 449.0, 1e30, -1e30, 448.0, -0.0, 0.0,
                  2.0 ** -10, -2.0 ** -10, 2.0 ** -10 * 1.0000001, -1e-30, 432.0, 431.9])
    got = e4m3_encode(x)
    exp = [0x7F, 0xFF, 0x7E, 0xFE, 0x7E, 0x7E, 0xFE, 0x7E, 0x80, 0x00,
           0x00,   # tie between 0 and 2^-9 -> even code 0x00
           0x80,   # negative tie to zero keeps the sign
           0x01, 0x80,
           0x7E,   # tie between 416 (0x7D) and 448 (0x7E) -> even 0x7E
           0x7D]
    assert list(got) == exp


def test_encode_matches_exact_rounder_on_boundaries():
    # every midpoint, and values one float64 ulp either side of it
    mids = [(MAGS[i] + MAGS[i + 1]) / 2 for i in range(126)]
    vals = []
    for m in mids:
        f = float(m)
        assert Fraction(f) == m
        vals += [f, np.nextafter(f, 0.0), np.nextafter(f, np.inf)]
    vals = np.array(vals + [-v for v in vals])
    got = e4m3_encode(vals)
    exp = [round_e4m3(Fraction(float(v)), v < 0 or (v == 0 and math.copysign(1, v) < 0))
           for v in vals]
    assert list(got) == exp


def test_encode_matches_exact_rounder_random():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(3000) * 50,
        np.exp2(rng.uniform(-14, 9.5, 3000)) * rng.choice([-1, 1], 3000),
    ])
    got = e4m3_encode(vals)
    exp = [round_e4m3(Fraction(float(v)), v < 0) for v in vals]
    assert list(got) == exp


def test_encode_matches_torch_cast_in_range():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even; it does not saturate,
    # so only values within the finite range are compared.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 30,
                        np.exp2(rng.uniform(-12, 8.7, 20000)) * rng.choice([-1, 1], 20000)])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), ref)

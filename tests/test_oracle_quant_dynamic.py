"""Pins for the oracle's dynamic per-head quantizer (oracle.quant_dynamic).

Independent of the formula as written: each head's largest element must encode to the
E4M3 maximum (448, sign kept); scaling the input by 2^k scales only the descales; an
all-zero head keeps its codes signed zeros with descale 1; a head of tiny values gets the
2^-126 floor; and the descale equals the exact rational amax/448 rounded to fp32.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import quant_dynamic, quant_static
from tests.exact_e4m3 import round_fp32


def _bf16(x32):
    """float32 array -> bf16 bit patterns (round to nearest even)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _x(seed=0, shape=(40, 5, 192), scale=None):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(shape).astype(np.float32)
    if scale is not None:
        z *= np.asarray(scale, dtype=np.float32)[None, :, None]
    return _bf16(z)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_max_element_maps_to_e4m3_max():
    x = _x(1, scale=[0.01, 1.0, 7.5, 300.0, 2.0 ** -100])
    codes, d = quant_dynamic(x)
    v = np.abs(_f(x))
    for h in range(x.shape[1]):
        at = v[:, h, :] == v[:, h, :].max()
        assert np.all((codes[:, h, :][at] & 0x7F) == 0x7E)
        # and nothing else saturates beyond it
        assert np.all((codes[:, h, :] & 0x7F) <= 0x7E)


def test_power_of_two_scaling_moves_only_the_descale():
    x = _x(2, scale=[0.5, 3.0, 40.0, 1e-3, 1e3])
    c0, d0 = quant_dynamic(x)
    for k in (-20, -3, 1, 9, 30):
        xs = _bf16(_f(x).astype(np.float32) * np.float32(2.0 ** k))
        c1, d1 = quant_dynamic(xs)
        assert np.array_equal(c0, c1), k
        assert np.array_equal(d1.astype(np.float64), d0.astype(np.float64) * 2.0 ** k), k


def test_zero_head_gives_signed_zeros_and_unit_descale():
    x = _x(3, shape=(16, 3, 128))
    x[:, 1, :] = 0
    x[::2, 1, ::3] = 0x8000  # -0
    codes, d = quant_dynamic(x)
    assert d[1] == np.float32(1.0)
    assert np.all(codes[:, 1, :][x[:, 1, :] == 0] == 0x00)
    assert np.all(codes[:, 1, :][x[:, 1, :] == 0x8000] == 0x80)


def test_tiny_head_descale_is_floored():
    x = _x(4, shape=(8, 2, 128), scale=[1.0, 2.0 ** -125])
    _, d = quant_dynamic(x)
    assert d[1] == np.float32(2.0 ** -126)
    assert d[0] > np.float32(2.0 ** -126)


def test_descale_is_exact_rational_rounding():
    x = _x(5, shape=(64, 6, 192), scale=[0.3, 1.7, 11.0, 0.02, 250.0, 5e-30])
    _, d = quant_dynamic(x)
    amax = np.abs(_f(x)).max(axis=(0, 2))
    for h in range(x.shape[1]):
        want = round_fp32(Fraction(float(amax[h])) / 448)
        assert Fraction(float(d[h])) == want, h


def test_codes_are_static_codes_with_the_dynamic_descale():
    x = _x(6, shape=(32, 4, 192), scale=[1.0, 0.25, 4.0, 100.0])
    codes, d = quant_dynamic(x)
    assert np.array_equal(codes, quant_static(x, d))


def test_rejects_non_finite_input():
    x = _x(7, shape=(4, 2, 128))
    x[0, 0, 0] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        quant_dynamic(x)

"""Pins for the oracle's static quantizer and descale arithmetic (oracle/quant.py).

Pinned against an exact-rational rounder written independently from the OCP
definition (tests/exact_e4m3.py) on every bf16 bit pattern, for ordinary,
power-of-two, workload and adversarial descales; and against exact fp32
rounding of amax / 448.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import amax_per_head, descale_from_amax, quant_static
from synth import make_workload
from tests.exact_e4m3 import quant_exact, round_fp32
from tests.quant_cases import adversarial_descales, all_bf16_patterns, standard_descales


def _exhaustive(descales):
    bits = all_bf16_patterns()
    h = len(descales)
    x = np.broadcast_to(bits[:, None, None], (65536, h, 1)).copy()
    d = np.array(descales, dtype=np.float32)
    got = quant_static(x, d)[:, :, 0]
    for j in range(h):
        exp = np.array([quant_exact(int(b), d[j]) for b in bits], dtype=np.uint8)
        bad = np.nonzero(got[:, j] != exp)[0]
        assert bad.size == 0, (float(d[j]), [hex(int(bits[i])) for i in bad[:5]])


def test_exhaustive_standard_descales():
    _exhaustive(standard_descales())


def test_adversarial_descales_exist_and_pass():
    adv = adversarial_descales()
    assert len(adv) >= 4
    _exhaustive(adv[:4])


def test_exhaustive_workload_descales():
    wl = make_workload("C1")
    cal = wl.calib()
    d = np.concatenate([descale_from_amax(amax_per_head(c)) for c in cal])
    _exhaustive(list(d[::6]))


def test_descale_from_amax_is_correctly_rounded_fp32():
    rng = np.random.default_rng(3)
    bits = rng.integers(0x0600, 0x7F7F, size=4000).astype(np.uint16)  # amax/448 stays fp32-normal
    amax = (bits.astype(np.uint32) << 16).view(np.float32)
    got = descale_from_amax(amax)
    for a, g in zip(amax, got):
        assert float(g) == round_fp32(Fraction(float(a)) / 448), float(a)


def test_descale_rejects_bad_amax():
    for bad in ([0.0], [-1.0], [np.inf], [np.nan]):
        with pytest.raises(ValueError):
            descale_from_amax(np.array(bad, dtype=np.float32))


def test_quant_rejects_bad_descales():
    x = np.zeros((2, 1, 4), dtype=np.uint16)
    for bad in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            quant_static(x, np.array([bad], dtype=np.float32))


def test_amax_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((7, 3, 5)) * 3).astype(np.float32)
    bits = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    got = amax_per_head(bits)
    for h in range(3):
        m = 0.0
        for t in range(7):
            for d in range(5):
                v = float(np.float32(np.uint32(int(bits[t, h, d]) << 16).view(np.float32)))
                m = max(m, abs(v))
        assert got[h] == m


def test_quant_shape_and_head_indexing():
    # head h must use descale[h]: quantize with distinct power-of-two descales, where the
    # quotient is exact, and compare with the codec applied per head
    from oracle import e4m3_encode
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((5, 4, 8)) * 10).astype(np.float32)
    bits = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    d = np.array([1.0, 0.5, 4.0, 0.125], dtype=np.float32)
    got = quant_static(bits, d)
    xv = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for h in range(4):
        assert np.array_equal(got[:, h], e4m3_encode(xv[:, h] / float(d[h])))

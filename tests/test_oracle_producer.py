"""Pins for the un-absorbed K/V producer oracle (oracle/producer.py).

Pinned against: an exact-rational (fractions.Fraction) round-to-nearest-even to
bf16, written from the definition; the float32 -> bf16 bit rounding on inputs
that are float32 values; a math.fsum brute force of the projection on tiny
inputs; closed forms (unit-vector weights gather latent columns, the rope part
is the same for every head and quantized with each head's scale) and an exact
power-of-two scaling invariant.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant_static
from oracle.producer import kv_produce, kv_project_bf16, rn_bf16_bits


def _rn_bf16_fraction(x: Fraction) -> int:
    """bf16 bits of the nearest-even bf16 value to the rational x (|x| below bf16 max)."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    e = -125  # smallest exponent with 8-bit significands of the normal range
    while a >= Fraction(2) ** e:
        e += 1
    while e > -125 and a < Fraction(2) ** (e - 1):
        e -= 1
    ulp = Fraction(2) ** (e - 8)
    q = a / ulp
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    f = float(val)
    bits = struct.unpack("<I", struct.pack("<f", f))[0]
    assert bits & 0xFFFF == 0
    return sign | (bits >> 16)


def _bf16(x):
    return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]


def test_rn_bf16_matches_exact_rationals():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000)))
    # exact ties and near ties around bf16 values, both parities, several binades
    for b in (0x3F80, 0x3F81, 0x4120, 0x4121, 0x0080, 0x0081, 0x7F00, 0xC2F7, 0x3400):
        lo = _bf16(b)
        hi = _bf16(b + 1)
        mid = (Fraction(lo) + Fraction(hi)) / 2
        for d in (Fraction(0), Fraction(1, 2 ** 60), -Fraction(1, 2 ** 60)):
            vals.append(float(mid + d * abs(Fraction(lo))))
    vals += [0.0, -0.0, 2.0 ** -130, -3 * 2.0 ** -134, 2.0 ** -133 * 2.5, 2.0 ** -126 * 0.75]
    got = rn_bf16_bits(np.array(vals))
    for v, g in zip(vals, got):
        want = _rn_bf16_fraction(Fraction(v)) if v != 0 else (0x8000 if math.copysign(1, v) < 0 else 0)
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_rn_bf16_equals_float32_bit_rounding_on_float32_inputs():
    rng = np.random.default_rng(1)
    b = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = b.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    u = f.view(np.uint32).astype(np.uint64)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(rn_bf16_bits(f.astype(np.float64)), want)


def _rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_projection_brute_force():
    rng = np.random.default_rng(2)
    T, H = 3, 2
    c = _rand_bf16(rng, (T, 512))
    w = _rand_bf16(rng, (H * 256, 512), 0.05)
    k_nope, v = kv_project_bf16(c, w, H)
    for t in range(T):
        for h in range(H):
            for f in list(range(0, 256, 17)) + [127, 128, 255]:
                row = w[h * 256 + f]
                exact = sum((Fraction(_bf16(c[t, i])) * Fraction(_bf16(row[i])) for i in range(512)),
                            Fraction(0))
                want = _rn_bf16_fraction(exact)
                got = k_nope[t, h, f] if f < 128 else v[t, h, f - 128]
                assert int(got) == want, (t, h, f)


def test_unit_vector_weights_gather_latent_columns():
    rng = np.random.default_rng(3)
    T, H = 5, 3
    c = _rand_bf16(rng, (T, 512))
    cols = rng.integers(0, 512, H * 256)
    w = np.zeros((H * 256, 512), dtype=np.uint16)
    w[np.arange(H * 256), cols] = 0x3F80  # 1.0
    k_nope, v = kv_project_bf16(c, w, H)
    g = c[:, cols].reshape(T, H, 256)
    # -0.0 * ... sums to +0.0: compare values, not bits, for zeros
    assert np.array_equal(k_nope, np.where(g[:, :, :128] == 0x8000, 0, g[:, :, :128]))
    assert np.array_equal(v, np.where(g[:, :, 128:] == 0x8000, 0, g[:, :, 128:]))


def test_rope_part_is_shared_and_quantized_per_head():
    rng = np.random.default_rng(4)
    T, H = 7, 4
    c = _rand_bf16(rng, (T, 512))
    pe = _rand_bf16(rng, (T, 64), 3.0)
    w = _rand_bf16(rng, (H * 256, 512), 0.05)
    dk = np.exp2(rng.uniform(-8, -4, H)).astype(np.float32)
    dv = np.exp2(rng.uniform(-8, -4, H)).astype(np.float32)
    k8, v8, k, v = kv_produce(c, pe, w, dk, dv)
    assert k8.shape == (T, H, 192) and v8.shape == (T, H, 128)
    for h in range(H):
        assert np.array_equal(k[:, h, 128:], pe)
        assert np.array_equal(k8[:, h, 128:], quant_static(pe[:, None, :], dk[h:h + 1])[:, 0])
    assert np.array_equal(v8, quant_static(v, dv))


def test_power_of_two_weight_scaling_is_exact():
    rng = np.random.default_rng(5)
    T, H = 4, 2
    c = _rand_bf16(rng, (T, 512))
    w = _rand_bf16(rng, (H * 256, 512), 0.05)
    w2 = (w.astype(np.uint32) + (w & 0x7FFF > 0) * (1 << 7)).astype(np.uint16)  # x2: exponent + 1
    k1, v1 = kv_project_bf16(c, w, H)
    k2, v2 = kv_project_bf16(c, w2, H)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(k2), 2 * f(k1)) and np.array_equal(f(v2), 2 * f(v1))


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        rn_bf16_bits(np.array([1.0, np.inf]))

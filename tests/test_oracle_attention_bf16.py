"""Pins for the oracle's BF16 attention (attention_varlen_bf16, attention_rows_bf16).

Pinned against: an explicit-loop brute force with math.fsum that decodes bf16
through struct (not through the oracle's decoder), the FP8 attention oracle on
inputs whose E4M3 values are exactly bf16 values (a separately pinned function),
a closed form (V = ones) and the selected-rows invariant.
"""

import math
import struct

import numpy as np
import pytest

from oracle import (attention_rows_bf16, attention_varlen, attention_varlen_bf16, e4m3_decode)

SCALE = 1.0 / math.sqrt(192)


def _bf16(rng, shape, sigma=1.0):
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do


def _val(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _case(rng, lens_q, lens_k, heads):
    tq, tk = sum(lens_q), sum(lens_k)
    q = _bf16(rng, (tq, heads, 192))
    k = _bf16(rng, (tk, heads, 192))
    v = _bf16(rng, (tk, heads, 128), 2.0)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return q, k, v, cu_q, cu_k


def _brute(q, k, v, cu_q, cu_k, scale, causal):
    tq, heads = q.shape[0], q.shape[1]
    out = np.zeros((tq, heads, 128))
    lse = np.full((heads, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        lq = int(cu_q[b + 1] - cu_q[b])
        lk = int(cu_k[b + 1] - cu_k[b])
        for h in range(heads):
            for i in range(lq):
                qi = int(cu_q[b]) + i
                logits, keys = [], []
                for j in range(lk):
                    if causal and j > i + (lk - lq):
                        continue
                    kj = int(cu_k[b]) + j
                    logits.append(scale * math.fsum(_val(q[qi, h, d]) * _val(k[kj, h, d])
                                                    for d in range(192)))
                    keys.append(kj)
                if not logits:
                    continue
                m = max(logits)
                w = [math.exp(s - m) for s in logits]
                l_ = math.fsum(w)
                for d in range(128):
                    out[qi, h, d] = math.fsum(wj * _val(v[kj, h, d]) for wj, kj in zip(w, keys)) / l_
                lse[h, qi] = m + math.log(l_)
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens", [([5, 1, 6], [5, 1, 6]), ([3, 5], [7, 5]), ([4, 2], [3, 0])])
def test_brute_force(causal, lens):
    rng = np.random.default_rng(101 + len(lens[0]) + 7 * int(causal))
    args = _case(rng, lens[0], lens[1], heads=2)
    out, lse = attention_varlen_bf16(*args, SCALE, causal)
    bo, bl = _brute(*args, SCALE, causal)
    assert np.allclose(out, bo, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-13)
    assert np.all(out[~fin.T] == 0)


def test_equals_fp8_oracle_on_exact_values():
    # E4M3 values (3 mantissa bits, exponents 2^-9 .. 2^8) are exact in bf16, so with unit
    # descales both oracles see identical inputs and must agree to the last bit
    rng = np.random.default_rng(5)
    lens = [9, 4]
    tq = tk = sum(lens)
    codes = [rng.integers(0, 256, size=(tq, 2, d)).astype(np.uint8) for d in (192, 192, 128)]
    for c in codes:
        c[(c & 0x7F) == 0x7F] = 0x3F
    bits = []
    for c in codes:
        f = e4m3_decode(c).astype(np.float32)
        assert np.array_equal(f.astype(np.float64), e4m3_decode(c))
        bits.append((f.view(np.uint32) >> 16).astype(np.uint16))
        assert np.all((f.view(np.uint32) & 0xFFFF) == 0)
    cu = np.array([0, 9, 13], dtype=np.int32)
    ones = np.ones(2, dtype=np.float32)
    for causal in (True, False):
        o8, l8 = attention_varlen(*codes, cu, cu, ones, ones, ones, 0.01, causal)
        ob, lb = attention_varlen_bf16(*bits, cu, cu, 0.01, causal)
        assert np.array_equal(o8, ob)
        assert np.array_equal(l8, lb)


def test_v_ones_gives_ones():
    rng = np.random.default_rng(9)
    q, k, v, cu_q, cu_k = _case(rng, [7, 3], [7, 3], heads=3)
    v[:] = 0x3F80  # bf16 1.0
    out, lse = attention_varlen_bf16(q, k, v, cu_q, cu_k, SCALE, True)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-15)
    assert np.all(np.isfinite(lse))


def test_rows_equals_full():
    rng = np.random.default_rng(13)
    args = _case(rng, [40, 9, 17], [40, 30, 17], heads=2)
    out, lse = attention_varlen_bf16(*args, SCALE, True)
    rows = np.array([0, 5, 39, 40, 48, 49, 65])
    ro, rl = attention_rows_bf16(*args, SCALE, True, rows)
    assert np.array_equal(ro, out[rows])
    assert np.array_equal(rl, lse[:, rows])

"""Pins for the oracle's LSE merge and chunked drivers (oracle/merge.py, oracle/chunked.py).

Pinned against: the two-segment closed form, the all-empty special case,
associativity, key-coverage of the segment plan by enumeration, and the
invariant that segmented-then-merged attention equals the unsegmented call
(for the chunked shapes of the 4K-over-64K and 128K workloads, scaled down).
"""

import math

import numpy as np
import pytest

from oracle import attention_varlen, chunked_context, merge_lse, segment_plan

SCALE = 1.0 / math.sqrt(192)


def test_two_segment_closed_form():
    rng = np.random.default_rng(0)
    o1, o2 = rng.standard_normal((2, 3, 2, 4))
    l1 = np.array([[0.3, -1.0, 2.0], [5.0, 0.0, -3.0]])
    l2 = np.array([[1.3, 4.0, -2.0], [-np.inf, 0.0, -3.0]])
    out, lse = merge_lse([o1, o2], [l1, l2])
    for h in range(2):
        for t in range(3):
            a, b = l1[h, t], l2[h, t]
            e1 = math.exp(a)
            e2 = 0.0 if b == -math.inf else math.exp(b)
            assert abs(lse[h, t] - math.log(e1 + e2)) < 1e-14
            exp = (e1 * o1[t, h] + e2 * o2[t, h]) / (e1 + e2)
            assert np.allclose(out[t, h], exp, rtol=1e-14, atol=1e-15)


def test_all_empty_segments():
    o = np.ones((2, 1, 3))
    l_ = np.full((1, 2), -np.inf)
    out, lse = merge_lse([o, 2 * o], [l_, l_])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_associativity():
    rng = np.random.default_rng(1)
    outs = [rng.standard_normal((5, 2, 4)) for _ in range(3)]
    lses = [rng.standard_normal((2, 5)) * 3 for _ in range(3)]
    o_all, l_all = merge_lse(outs, lses)
    o_ab, l_ab = merge_lse(outs[:2], lses[:2])
    o2, l2 = merge_lse([o_ab, outs[2]], [l_ab, lses[2]])
    assert np.allclose(o_all, o2, rtol=1e-13)
    assert np.allclose(l_all, l2, rtol=1e-13)


@pytest.mark.parametrize("lq,lk,seg,causal", [(4, 20, 4, True), (16, 16, 4, True), (7, 23, 5, True),
                                              (10, 10, 3, True), (6, 13, 4, False)])
def test_plan_covers_each_visible_key_once(lq, lk, seg, causal):
    plan = segment_plan(lq, lk, seg, causal)
    seen = np.zeros((lq, lk), dtype=int)
    rows = []
    for r0, r1, parts in plan:
        rows += list(range(r0, r1))
        for k0, k1, c in parts:
            for i in range(r0, r1):
                for j in range(k0, k1):
                    if c and (j - k0) > (i - r0) + ((k1 - k0) - (r1 - r0)):
                        continue
                    seen[i, j] += 1
    assert rows == list(range(lq))
    off = lk - lq
    for i in range(lq):
        for j in range(lk):
            vis = (not causal) or j <= i + off
            assert seen[i, j] == (1 if vis else 0), (i, j)


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F
    return c


@pytest.mark.parametrize("lq,lk,seg", [(16, 80, 16), (64, 64, 16), (40, 40, 16), (9, 30, 7)])
def test_segmented_equals_unsegmented(lq, lk, seg):
    rng = np.random.default_rng(lq * 1000 + lk)
    h = 2
    q, k, v = _codes(rng, (lq, h, 192)), _codes(rng, (lk, h, 192)), _codes(rng, (lk, h, 128))
    dq = np.full(h, 2.0 ** -7, np.float32)
    dk = np.full(h, 2.0 ** -6, np.float32)
    dv = np.full(h, 0.25, np.float32)
    ref_o, ref_l = attention_varlen(q, k, v, [0, lq], [0, lk], dq, dk, dv, SCALE, True)
    o, l_ = chunked_context(q, k, v, dq, dk, dv, SCALE, seg, True)
    assert np.allclose(o, ref_o, rtol=1e-12, atol=1e-14)
    assert np.allclose(l_, ref_l, rtol=1e-12)

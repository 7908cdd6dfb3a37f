"""Pins for the oracle's attention (oracle/attention.py).

Pinned against: an explicit-loop brute force with math.fsum on tiny inputs
(written from the definition, not from the vectorized code), closed forms
(V = ones, a length-1 sequence, Q = 0, two keys), and invariants (permutation
of packed sequences, head independence, last causal row = non-causal row,
empty rows, selected rows = full result).
"""

import math

import numpy as np
import pytest

from oracle import attention_rows, attention_varlen, e4m3_decode

SCALE = 1.0 / math.sqrt(192)


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes in attention inputs
    return c


def _case(rng, lens_q, lens_k, heads):
    tq, tk = sum(lens_q), sum(lens_k)
    q = _rand_codes(rng, (tq, heads, 192))
    k = _rand_codes(rng, (tk, heads, 192))
    v = _rand_codes(rng, (tk, heads, 128))
    dq = (np.exp2(rng.uniform(-8, -5, heads))).astype(np.float32)
    dk = (np.exp2(rng.uniform(-8, -5, heads))).astype(np.float32)
    dv = (np.exp2(rng.uniform(-3, 0, heads))).astype(np.float32)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return q, k, v, cu_q, cu_k, dq, dk, dv


def _brute(q, k, v, cu_q, cu_k, dq, dk, dv, scale, causal):
    tab = [float(x) for x in e4m3_decode(np.arange(256, dtype=np.uint8))]
    tq, heads = q.shape[0], q.shape[1]
    out = np.zeros((tq, heads, 128))
    lse = np.full((heads, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        lq = int(cu_q[b + 1] - cu_q[b])
        lk = int(cu_k[b + 1] - cu_k[b])
        for h in range(heads):
            for i in range(lq):
                qi = int(cu_q[b]) + i
                logits = []
                keys = []
                for j in range(lk):
                    if causal and j > i + (lk - lq):
                        continue
                    kj = int(cu_k[b]) + j
                    s = math.fsum(tab[q[qi, h, d]] * float(dq[h]) * tab[k[kj, h, d]] * float(dk[h])
                                  for d in range(192))
                    logits.append(scale * s)
                    keys.append(kj)
                if not logits:
                    continue
                m = max(logits)
                w = [math.exp(s - m) for s in logits]
                l_ = math.fsum(w)
                for d in range(128):
                    out[qi, h, d] = math.fsum(wj * tab[v[kj, h, d]] * float(dv[h])
                                              for wj, kj in zip(w, keys)) / l_
                lse[h, qi] = m + math.log(l_)
    return out, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens", [([5, 1, 7], [5, 1, 7]), ([3, 6], [8, 6]), ([6, 2], [4, 0])])
def test_brute_force(causal, lens):
    rng = np.random.default_rng(17 + len(lens[0]) + int(causal))
    args = _case(rng, lens[0], lens[1], heads=2)
    out, lse = attention_varlen(*args, SCALE, causal)
    bo, bl = _brute(*args, SCALE, causal)
    assert np.allclose(out, bo, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)


def test_v_ones_gives_ones():
    rng = np.random.default_rng(1)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [9, 4], [9, 6], heads=3)
    v[:] = 0x38  # 1.0
    dv[:] = 1.0
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    assert np.allclose(out, 1.0, atol=1e-14)


def test_length_one_sequence():
    rng = np.random.default_rng(2)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [1], [1], heads=2)
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    for h in range(2):
        vd = e4m3_decode(v[0, h]) * float(dv[h])
        assert np.allclose(out[0, h], vd, rtol=1e-15)
        s = SCALE * float(np.dot(e4m3_decode(q[0, h]) * float(dq[h]), e4m3_decode(k[0, h]) * float(dk[h])))
        assert abs(lse[h, 0] - s) < 1e-12


def test_q_zero_closed_form():
    rng = np.random.default_rng(3)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [6], [10], heads=2)
    q[:] = 0
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    for h in range(2):
        vd = e4m3_decode(v[:, h]) * float(dv[h])
        for i in range(6):
            n = i + (10 - 6) + 1
            assert np.allclose(out[i, h], vd[:n].mean(axis=0), rtol=1e-13, atol=1e-15)
            assert abs(lse[h, i] - math.log(n)) < 1e-13


def test_two_keys_sigmoid():
    # two keys with logits s0, s1: weight of key 1 is the logistic function of s1 - s0
    q = np.zeros((1, 1, 192), dtype=np.uint8)
    k = np.zeros((2, 1, 192), dtype=np.uint8)
    v = np.zeros((2, 1, 128), dtype=np.uint8)
    q[0, 0, 0] = 0x38   # 1.0
    k[0, 0, 0] = 0x30   # 0.5
    k[1, 0, 0] = 0x40   # 2.0
    v[0, 0, :] = 0x00   # 0
    v[1, 0, :] = 0x38   # 1
    one = np.ones(1, dtype=np.float32)
    out, lse = attention_varlen(q, k, v, [0, 1], [0, 2], one, one, one, 1.0, False)
    w1 = 1.0 / (1.0 + math.exp(-(2.0 - 0.5)))
    assert abs(out[0, 0, 5] - w1) < 1e-15
    assert abs(lse[0, 0] - math.log(math.exp(0.5) + math.exp(2.0))) < 1e-14


def test_permutation_of_packed_sequences():
    rng = np.random.default_rng(4)
    lens = [7, 3, 12, 5]
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, lens, lens, heads=2)
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    perm = [2, 0, 3, 1]
    segs = [(cu_q[b], cu_q[b + 1]) for b in perm]
    idx = np.concatenate([np.arange(a, b) for a, b in segs])
    lens_p = [lens[b] for b in perm]
    cu_p = np.concatenate([[0], np.cumsum(lens_p)]).astype(np.int32)
    out_p, lse_p = attention_varlen(q[idx], k[idx], v[idx], cu_p, cu_p, dq, dk, dv, SCALE, True)
    assert np.array_equal(out_p, out[idx])
    assert np.array_equal(lse_p, lse[:, idx])


def test_head_independence():
    rng = np.random.default_rng(5)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [8, 5], [8, 5], heads=4)
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    sel = [3, 1]
    o2, l2 = attention_varlen(q[:, sel], k[:, sel], v[:, sel], cu_q, cu_k, dq[sel], dk[sel], dv[sel],
                              SCALE, True)
    assert np.array_equal(o2, out[:, sel])
    assert np.array_equal(l2, lse[sel])


def test_last_causal_row_equals_noncausal():
    rng = np.random.default_rng(6)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [11], [11], heads=2)
    oc, lc = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    on, ln = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, False)
    assert np.allclose(oc[-1], on[-1], rtol=1e-14, atol=1e-15)
    assert np.allclose(lc[:, -1], ln[:, -1], rtol=1e-14)
    # and the first causal row sees exactly one key
    vd0 = e4m3_decode(v[0]) * dv[:, None].astype(np.float64)
    assert np.allclose(oc[0], vd0, rtol=1e-15)


def test_empty_rows_when_lq_exceeds_lk():
    rng = np.random.default_rng(7)
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, [6], [2], heads=1)
    out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, True)
    # bottom-right: row i sees keys j <= i - 4; rows 0..3 see none
    assert np.all(out[:4] == 0) and np.all(np.isneginf(lse[:, :4]))
    assert np.all(np.isfinite(lse[:, 4:]))


def test_rows_equals_full():
    rng = np.random.default_rng(8)
    lens = [9, 14, 3]
    q, k, v, cu_q, cu_k, dq, dk, dv = _case(rng, lens, [12, 14, 5], heads=3)
    for causal in (True, False):
        out, lse = attention_varlen(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, causal)
        rows = np.array([0, 5, 9, 10, 22, 25, 24, 1])
        o, l_ = attention_rows(q, k, v, cu_q, cu_k, dq, dk, dv, SCALE, causal, rows)
        assert np.allclose(o, out[rows], rtol=1e-13, atol=1e-15)
        assert np.allclose(l_, lse[:, rows], rtol=1e-13)

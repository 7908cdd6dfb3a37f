"""CPU checks of the parity gates' own helpers: the bf16 spacing, the stratified row
sample, and the per-row LSE error scale R_i against explicit loops."""

import math

import numpy as np

import oracle
from synth.inputs import make_random
from tests.parity import lse_scale_fp8, stratified_rows, ulp_bf16


def test_ulp_bf16():
    assert ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7
    assert ulp_bf16(np.array([1.99]))[0] == 2.0 ** -7
    assert ulp_bf16(np.array([-8.0]))[0] == 2.0 ** -4
    assert ulp_bf16(np.array([0.02]))[0] == 2.0 ** -13
    # the spacing is that of consecutive bf16 bit patterns
    bits = np.array([0x3F80, 0x4100, 0x3C00, 0x4480], np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    nxt = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(ulp_bf16(v), nxt - v)


def test_stratified_rows_cover_every_block_and_lane():
    rows = stratified_rows(32768, 3, extra=[0, 32767])
    blocks = rows // 32
    assert np.array_equal(np.unique(blocks), np.arange(1024))
    lanes = np.bincount(rows % 32, minlength=32)
    assert lanes.min() >= 32  # every lane position, about equally often
    tail = stratified_rows(100, 1)  # a ragged last block stays in range
    assert tail.max() < 100 and len(np.unique(tail // 32)) == 4


def test_row_lse_scale_matches_loops():
    wl = make_random(77, [9, 5], [12, 5], causal=True, heads=2)
    ds = [oracle.descale_from_amax(oracle.amax_per_head(x)) for x in (wl.q, wl.k, wl.v)]
    q8, k8, v8 = (oracle.quant_static(x, d) for x, d in zip((wl.q, wl.k, wl.v), ds))
    _, lse = oracle.attention_varlen(q8, k8, v8, wl.cu_seqlens_q, wl.cu_seqlens_k, *ds,
                                     wl.softmax_scale, True)
    rows = np.arange(wl.total_q)
    r = lse_scale_fp8(q8, k8, ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k, rows,
                      wl.softmax_scale, True, lse)
    dec = oracle.e4m3_decode
    for b in range(2):
        q0, q1 = wl.cu_seqlens_q[b], wl.cu_seqlens_q[b + 1]
        k0, k1 = wl.cu_seqlens_k[b], wl.cu_seqlens_k[b + 1]
        lq, lk = q1 - q0, k1 - k0
        for h in range(2):
            for i in range(lq):
                qi = dec(q8[q0 + i, h]) * float(ds[0][h])
                acc = []
                for j in range(lk):
                    if j > i + (lk - lq):
                        continue
                    kj = dec(k8[k0 + j, h]) * float(ds[1][h])
                    s = wl.softmax_scale * math.fsum(qi * kj)
                    a = wl.softmax_scale * math.fsum(np.abs(qi * kj))
                    acc.append(math.exp(s - lse[h, q0 + i]) * a)
                assert abs(r[h, q0 + i] - math.fsum(acc)) <= 1e-12 * max(1.0, abs(r[h, q0 + i]))

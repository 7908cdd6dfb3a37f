"""Checks of the shared seeded input generators (synth/)."""

import numpy as np
import pytest

from synth import CONFIGS, D_QK, D_V, N_HEADS, f32_to_bf16_bits, make_workload
from synth.inputs import _pairs, make_random


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 7,
                        (rng.integers(0, 2 ** 32, 50000, dtype=np.uint64)).astype(np.uint32).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_workload_c1_shapes_and_determinism():
    a = make_workload("C1")
    b = make_workload("C1")
    assert a.q.shape == (128, N_HEADS, D_QK) and a.k.shape == (128, N_HEADS, D_QK)
    assert a.v.shape == (128, N_HEADS, D_V)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert np.array_equal(a.calib()[0], b.calib()[0])
    assert not np.array_equal(a.q, a.calib()[0])
    assert a.factors.min() >= 0.25 and a.factors.max() <= 4.0


def test_workload_c2_structure():
    w = make_workload("C2")
    lens = np.diff(w.cu_seqlens_q)
    assert lens.shape == (8,) and lens.min() >= 256 and lens.max() <= 4096
    assert w.cu_seqlens_q.dtype == np.int32
    assert [m.sum() for m in w.outlier_mask] == [2, 2, 2]


def test_pairs_brute_force():
    for lq in range(0, 9):
        for lk in range(0, 9):
            n = sum(1 for i in range(lq) for j in range(lk) if j <= i + (lk - lq))
            assert _pairs(lq, lk, True) == n, (lq, lk)
            assert _pairs(lq, lk, False) == lq * lk


def test_c3_flop_count():
    spec = CONFIGS["C3"]
    assert spec["lens"] == [32768]
    w = make_random(1, [16, 5], [20, 5])
    assert w.visible_pairs() == _pairs(16, 20, True) + _pairs(5, 5, True)

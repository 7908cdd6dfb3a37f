"""GPU parity of the BF16 comparator prefill against the fp64 oracle on bf16 inputs.

Same gates as the FP8 path (rel-RMS 1e-2; max-abs 2e-2 in absolute units, or one bf16
ulp of the reference where that is larger, and in V-scale units; LSE within
2^-9 + 1e-3 + 2^-12 R_i, here with R_i from the bf16 values). Element-wise on
small shapes spanning several 128-row query tiles and 32-key tiles with ragged
tails (causal and non-causal, Lq != Lk both ways, empty sequences), the full C2
workload, 1,024 stratified rows of the 32K causal workload in the benchmark's launch
(one per 32-row wave block of every 128-row query tile), and
invariants (bitwise determinism, V = ones). The last test compares the FP8 and
the BF16 path against the same bf16 oracle, the accuracy side of the comparison.
"""

import numpy as np
import pytest

import oracle
from synth import make_workload
from synth.inputs import make_random
from tests.gpu_helpers import (dev, dev_bf16, gpu_prefill, host, oracle_attention, oracle_codes,
                               oracle_descales)
from tests.parity import (assert_attention_parity, attention_errors, bf16_bits_to_f64,
                          lse_scale_bf16, record, sigma_v, stratified_rows)

pytestmark = pytest.mark.gpu


def _r(wl, rows, ref_l):
    return lse_scale_bf16(wl.q, wl.k, wl.cu_seqlens_q, wl.cu_seqlens_k, rows, wl.softmax_scale,
                          wl.causal, ref_l)


def _run(B, wl, q=None, k=None, v=None, causal=None):
    q = wl.q if q is None else q
    k = wl.k if k is None else k
    v = wl.v if v is None else v
    causal = wl.causal if causal is None else causal
    out, lse = B.prefill_varlen_bf16(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev(wl.cu_seqlens_q),
                                     dev(wl.cu_seqlens_k), wl.max_seqlen_q, wl.max_seqlen_k,
                                     wl.softmax_scale, causal)
    return bf16_bits_to_f64(host(out)), host(lse).astype(np.float64)


def _check(B, wl, label):
    out, lse = _run(B, wl)
    ref_o, ref_l = oracle.attention_varlen_bf16(wl.q, wl.k, wl.v, wl.cu_seqlens_q, wl.cu_seqlens_k,
                                                wl.softmax_scale, wl.causal)
    errs = attention_errors(out, ref_o, lse, ref_l, sigma_v(wl), _r(wl, np.arange(wl.total_q), ref_l))
    print(label, errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label)
    empty = ~np.isfinite(ref_l)
    if empty.any():
        assert np.all(out.transpose(1, 0, 2)[empty] == 0.0)
    return errs


CASES = [
    ("ragged_causal", [1, 5, 31, 33, 127, 128, 129, 300, 64, 0], None, True),
    ("ragged_noncausal", [1, 5, 31, 33, 127, 128, 129, 300, 64, 0], None, False),
    ("lk_gt_lq_causal", [100, 37, 200, 256], [300, 37, 64, 700], True),
    ("lk_gt_lq_noncausal", [100, 37, 200, 256], [300, 37, 64, 700], False),
    ("lq_gt_lk_causal", [300, 64, 97], [100, 0, 33], True),
    ("single_long", [777], None, True),
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
def test_bf16_small_cases(gpu_lib, case):
    name, lq, lk, causal = CASES[case]
    wl = make_random(300 + case, lq, lk, causal=causal, outliers=True)
    _check(gpu_lib, wl, "bf16 " + name)


def test_bf16_c1_c2_full(gpu_lib):
    _check(gpu_lib, make_workload("C1"), "bf16 C1")
    _check(gpu_lib, make_workload("C2"), "bf16 C2")


def test_bf16_c3_sampled_rows(gpu_lib):
    """32K causal at full size (one sequence, the XCD-aware block order); 1,024 stratified
    rows plus the edges."""
    B = gpu_lib
    wl = make_workload("C3")
    out, lse = _run(B, wl)
    L = wl.total_q
    rows = stratified_rows(L, 4, extra=[0, 1, 31, 32, 127, 128, 129, L - 129, L - 33, L - 1])
    assert len(rows) >= 1024
    ref_o, ref_l = oracle.attention_rows_bf16(wl.q, wl.k, wl.v, wl.cu_seqlens_q, wl.cu_seqlens_k,
                                              wl.softmax_scale, True, rows)
    errs = attention_errors(out[rows], ref_o, lse[:, rows], ref_l, sigma_v(wl), _r(wl, rows, ref_l))
    print("bf16 C3 sampled", errs, flush=True)
    record("bf16 C3 stratified rows", errs)
    assert_attention_parity(errs, "bf16 C3 sampled", absolute=True)


def test_bf16_determinism_and_v_ones(gpu_lib):
    B = gpu_lib
    wl = make_random(21, [300, 129, 64, 1000, 7], causal=True, outliers=True)
    o1, l1 = _run(B, wl)
    o2, l2 = _run(B, wl)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ones = np.full_like(wl.v, 0x3F80)  # bf16 1.0
    o3, l3 = _run(B, wl, v=ones)
    # the normalisation divides by the sum of the same rounded weights
    assert np.max(np.abs(o3 - 1.0)) <= 2.0 ** -8
    assert np.array_equal(l3, l1)


def test_fp8_and_bf16_against_the_bf16_oracle(gpu_lib):
    """Accuracy side of the comparison: the FP8 path (quantized inputs) and the BF16 path,
    both against exact attention on the unquantized bf16 inputs. The BF16 path must be the
    closer one; the FP8 path's distance is dominated by input quantization."""
    B = gpu_lib
    wl = make_workload("C2")
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    out8, lse8 = gpu_prefill(B, wl, [dev(c) for c in codes], [dev(d) for d in ds])
    out8 = bf16_bits_to_f64(host(out8))
    out16, lse16 = _run(B, wl)
    ref_o, ref_l = oracle.attention_varlen_bf16(wl.q, wl.k, wl.v, wl.cu_seqlens_q, wl.cu_seqlens_k,
                                                wl.softmax_scale, wl.causal)
    q8_o, _ = oracle_attention(wl, codes, ds)
    r = _r(wl, np.arange(wl.total_q), ref_l)
    e8 = attention_errors(out8, ref_o, host(lse8).astype(np.float64), ref_l, sigma_v(wl), r)
    e16 = attention_errors(out16, ref_o, lse16, ref_l, sigma_v(wl), r)
    eq = attention_errors(q8_o, ref_o, ref_l, ref_l, sigma_v(wl), r)
    print("vs bf16 oracle: fp8 path", e8, "bf16 path", e16, "exact on fp8 inputs", eq, flush=True)
    record("C2 fp8 path vs bf16 oracle", e8)
    record("C2 bf16 path vs bf16 oracle", e16)
    record("C2 exact attention on fp8 inputs vs bf16 oracle", eq)
    assert e16["rel_rms"] < e8["rel_rms"]
    assert e16["rel_rms"] <= 1e-2

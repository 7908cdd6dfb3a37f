"""GPU parity of the FP8 varlen prefill against the fp64 oracle.

Element-wise on small shapes that span several 256-row query tiles and
64-key tiles with ragged tails (causal and non-causal, Lq != Lk both ways,
empty sequences, sequences without keys, both block orders, 204 packed sequences);
the full small workloads; 1,024 rows of the 32K-token
causal workload in the launch configuration the benchmark times (one in every 32-row
block, so every query tile and wave of the launch, with the row within the block
spread over all lanes); and GPU-side
invariants (run-to-run bitwise determinism, permutation of packed sequences,
exact power-of-two V scaling, V = ones); a lazy rescale forced on every tile and
extreme softmax scales; and the 4-wave kernel that small grids run, bitwise against the
8-wave one on every small case.
"""

import dataclasses

import numpy as np
import pytest

import oracle
from synth import make_workload
from synth.inputs import make_random
from tests.gpu_helpers import (dev, gpu_descales, gpu_prefill, gpu_quant, host, oracle_attention,
                               oracle_codes, oracle_descales)
from tests.parity import (assert_attention_parity, attention_errors, bf16_bits_to_f64, lse_scale_fp8,
                          record, sigma_v, stratified_rows)

pytestmark = pytest.mark.gpu


def _run_codes(B, wl, codes, ds_np, causal=None):
    dcodes = [dev(c) for c in codes]
    dds = [dev(d) for d in ds_np]
    out, lse = gpu_prefill(B, wl, dcodes, dds, causal)
    return bf16_bits_to_f64(host(out)), host(lse).astype(np.float64)


def _r_all(wl, codes, ds, ref_l, causal=None):
    causal = wl.causal if causal is None else causal
    return lse_scale_fp8(codes[0], codes[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k,
                         np.arange(wl.total_q), wl.softmax_scale, causal, ref_l)


def _check(B, wl, causal=None, label=""):
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    out, lse = _run_codes(B, wl, codes, ds, causal)
    ref_o, ref_l = oracle_attention(wl, codes, ds, causal)
    errs = attention_errors(out, ref_o, lse, ref_l, sigma_v(wl), _r_all(wl, codes, ds, ref_l, causal))
    print(label, errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label)
    # rows without a visible key are exactly zero
    empty = ~np.isfinite(ref_l)  # [H, T]
    if empty.any():
        assert np.all(out.transpose(1, 0, 2)[empty] == 0.0)
    return errs


CASES = [
    ("ragged_causal", [1, 5, 127, 128, 129, 300, 64, 0], None, True, 12),
    ("ragged_noncausal", [1, 5, 127, 128, 129, 300, 64, 0], None, False, 12),
    ("lk_gt_lq_causal", [100, 37, 200, 256], [300, 37, 64, 700], True, 12),
    ("lk_gt_lq_noncausal", [100, 37, 200, 256], [300, 37, 64, 700], False, 12),
    ("single_long", [777], None, True, 12),
    # more queries than keys: bottom-right causal rows before the first key see nothing,
    # and a sequence without keys leaves all its rows empty (zero output, LSE -inf)
    ("lq_gt_lk_causal", [300, 129, 64, 5], [100, 0, 64, 3], True, 12),
    ("lq_gt_lk_noncausal", [300, 129, 64, 5], [100, 0, 64, 3], False, 12),
    # one sequence with a head count that is not a multiple of 4 and an odd number of
    # query tiles: the plain heaviest-first block order instead of the XCD-aware one
    ("one_seq_5_heads_odd_tiles", [600], None, True, 5),
    # the XCD-aware order with 4 half-heads per XCD, and a single head
    ("one_seq_16_heads", [1024], None, True, 16),
    ("one_head_lk_gt_lq", [700], [900], True, 1),
]


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
def test_prefill_small_cases(gpu_lib, case):
    name, lq, lk, causal, heads = CASES[case]
    wl = make_random(100 + case, lq, lk, causal=causal, heads=heads, outliers=True)
    _check(gpu_lib, wl, label=name)


@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[0] for c in CASES])
def test_small_grid_kernel_matches_the_8_wave_kernel(gpu_lib, case, monkeypatch):
    """Every case above is a grid of at most one 256-row workgroup per CU: with
    MLA_FP8_PREFILL_SMALL_GRID=1 it runs on the 4-wave workgroups of 128 rows, with 0 on
    the 8-wave kernel. Each query row takes the same arithmetic in both (one wave of 32
    rows, the same tiles in the same order), so the outputs and LSEs are bitwise equal."""
    B = gpu_lib
    name, lq, lk, causal, heads = CASES[case]
    wl = make_random(100 + case, lq, lk, causal=causal, heads=heads, outliers=True)
    ds = oracle_descales(wl)
    dcodes = [dev(c) for c in oracle_codes(wl, ds)]
    dds = [dev(d) for d in ds]
    monkeypatch.setenv("MLA_FP8_PREFILL_SMALL_GRID", "1")
    out4, lse4 = (host(x) for x in gpu_prefill(B, wl, dcodes, dds))
    monkeypatch.setenv("MLA_FP8_PREFILL_SMALL_GRID", "0")
    out8, lse8 = (host(x) for x in gpu_prefill(B, wl, dcodes, dds))
    assert np.array_equal(out4, out8), name
    assert np.array_equal(lse4.view(np.uint32), lse8.view(np.uint32)), name


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_many_short_sequences(gpu_lib, causal):
    """200 packed sequences of 0-40 query tokens plus four of 200-300 (key lengths drawn
    separately when non-causal): the (sequence, head) pairs of every query tile index in
    their rotated order, most of the grid's workgroups past a short sequence's end, and
    sequences without queries or keys."""
    rng = np.random.default_rng(77 if causal else 78)
    lq = np.concatenate([rng.integers(0, 41, 200), [200, 256, 257, 300]])
    rng.shuffle(lq)
    lk = None if causal else rng.integers(0, 60, lq.shape[0])
    wl = make_random(300 + int(causal), lq, lk, causal=causal, heads=12, outliers=True)
    _check(gpu_lib, wl, label=f"many_short_{'causal' if causal else 'noncausal'}")


def test_prefill_c1_full_pipeline(gpu_lib):
    """Workload C1 end to end through the library: calibration, one-launch quant, prefill."""
    B = gpu_lib
    wl = make_workload("C1")
    d_gpu = gpu_descales(B, wl)
    d_ref = oracle_descales(wl)
    assert all(np.array_equal(a, b) for a, b in zip(d_gpu, d_ref))
    codes, dds = gpu_quant(B, wl, d_gpu)
    ref_codes = oracle_codes(wl, d_ref)
    assert all(np.array_equal(host(c), r) for c, r in zip(codes, ref_codes))
    out, lse = gpu_prefill(B, wl, codes, dds)
    ref_o, ref_l = oracle_attention(wl, ref_codes, d_ref)
    errs = attention_errors(bf16_bits_to_f64(host(out)), ref_o, host(lse).astype(np.float64), ref_l,
                            sigma_v(wl), _r_all(wl, ref_codes, d_ref, ref_l))
    print("C1", errs, flush=True)
    record("C1 full", errs)
    assert_attention_parity(errs, "C1", absolute=True)


def test_prefill_c2_full(gpu_lib):
    _check(gpu_lib, make_workload("C2"), label="C2")


def test_c2_runs_the_4_wave_kernel_bitwise_like_the_8_wave_one(gpu_lib, monkeypatch):
    """The C2 mix (8 sequences of 808-3,975 tokens, a third of its grid padding) runs on
    128-row workgroups; with MLA_FP8_PREFILL_SMALL_GRID=0 on the 8-wave kernel. Bitwise
    equal outputs and LSEs."""
    B = gpu_lib
    wl = make_workload("C2")
    ds = oracle_descales(wl)
    dcodes = [dev(c) for c in oracle_codes(wl, ds)]
    dds = [dev(d) for d in ds]
    monkeypatch.delenv("MLA_FP8_PREFILL_SMALL_GRID", raising=False)
    out4, lse4 = (host(x) for x in gpu_prefill(B, wl, dcodes, dds))
    monkeypatch.setenv("MLA_FP8_PREFILL_SMALL_GRID", "0")
    out8, lse8 = (host(x) for x in gpu_prefill(B, wl, dcodes, dds))
    assert np.array_equal(out4, out8)
    assert np.array_equal(lse4.view(np.uint32), lse8.view(np.uint32))


def test_prefill_c3_sampled_rows(gpu_lib):
    """32K causal at full size, same launch as the benchmark; oracle on 1,024 stratified rows
    (one per 32-row wave block of every 256-row query tile) plus the edges."""
    B = gpu_lib
    wl = make_workload("C3")
    ds = gpu_descales(B, wl)
    codes, dds = gpu_quant(B, wl, ds)
    out, lse = gpu_prefill(B, wl, codes, dds)
    L = wl.total_q
    rows = stratified_rows(L, 3, extra=[0, 1, 63, 64, 127, 128, 129, L - 129, L - 128, L - 1])
    assert len(rows) >= 1024
    c_np = [host(c) for c in codes]
    ref_o, ref_l = oracle.attention_rows(c_np[0], c_np[1], c_np[2], wl.cu_seqlens_q,
                                         wl.cu_seqlens_k, ds[0], ds[1], ds[2], wl.softmax_scale,
                                         True, rows)
    got_o = bf16_bits_to_f64(host(out[rows]))
    got_l = host(lse[:, rows]).astype(np.float64)
    r = lse_scale_fp8(c_np[0], c_np[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k, rows,
                      wl.softmax_scale, True, ref_l)
    errs = attention_errors(got_o, ref_o, got_l, ref_l, sigma_v(wl), r)
    print("C3 sampled", errs, flush=True)
    record("C3 stratified rows", errs)
    assert_attention_parity(errs, "C3 sampled", absolute=True)
    # the quantizer bytes at full size are bit-exact as well (sampled tokens)
    rng = np.random.default_rng(3)
    d_ref = oracle_descales(wl)
    assert all(np.array_equal(a, b) for a, b in zip(ds, d_ref))
    toks = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 2000)]))
    for c, x, d in zip(c_np, (wl.q, wl.k, wl.v), d_ref):
        assert np.array_equal(c[toks], oracle.quant_static(x[toks], d))


def test_determinism_and_permutation(gpu_lib):
    B = gpu_lib
    lens = [300, 129, 64, 1000, 7]
    wl = make_random(5, lens, causal=True)
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    o1, l1 = _run_codes(B, wl, codes, ds)
    o2, l2 = _run_codes(B, wl, codes, ds)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = [3, 0, 4, 2, 1]
    cu = wl.cu_seqlens_q
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in perm])
    wl_p = make_random(5, [lens[b] for b in perm], causal=True)
    codes_p = [c[idx] for c in codes]
    op, lp = _run_codes(B, wl_p, codes_p, ds)
    assert np.array_equal(op, o1[idx]) and np.array_equal(lp, l1[:, idx])


def test_power_of_two_v_scale_is_exact(gpu_lib):
    B = gpu_lib
    wl = make_random(9, [200, 77], causal=True)
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    o1, l1 = _run_codes(B, wl, codes, ds)
    ds2 = [ds[0], ds[1], (ds[2] * 2).astype(np.float32)]
    o2, l2 = _run_codes(B, wl, codes, ds2)
    assert np.array_equal(o2, 2 * o1) and np.array_equal(l1, l2)


def test_v_ones(gpu_lib):
    B = gpu_lib
    wl = make_random(11, [150, 64, 9], [150, 100, 9], causal=True)
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    codes[2] = np.full_like(codes[2], 0x38)
    ds[2] = np.ones_like(ds[2])
    out, lse = _run_codes(B, wl, codes, ds)
    assert np.max(np.abs(out - 1.0)) <= 4e-3


def _check_own_scales(B, wl, label, max_abs_gate=True):
    # descales from the data itself (the tensors below are reshaped after generation)
    ds = [oracle.descale_from_amax(oracle.amax_per_head(x)) for x in (wl.q, wl.k, wl.v)]
    codes = oracle_codes(wl, ds)
    out, lse = _run_codes(B, wl, codes, ds)
    ref_o, ref_l = oracle_attention(wl, codes, ds)
    errs = attention_errors(out, ref_o, lse, ref_l, sigma_v(wl), _r_all(wl, codes, ds, ref_l))
    print(label, errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label, max_abs=max_abs_gate)


def test_rescale_on_every_tile(gpu_lib):
    """Logits that grow by ~12 (base 2) per 64-key tile along the keys: every row's running
    maximum moves past the lazy-rescale slack on every tile it sees, so O and the row sum
    are rescaled on each iteration."""
    from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits

    wl = make_random(4242, [300, 517], None, causal=True)
    q = bf16_bits_to_f32(wl.q)
    k = bf16_bits_to_f32(wl.k)
    q[:, :, 0] = 4.0
    step = 12.0 / (np.log2(np.e) * wl.softmax_scale * 4.0)  # key-dim-0 rise per 64 keys
    for b in range(wl.batch):
        k0, k1 = int(wl.cu_seqlens_k[b]), int(wl.cu_seqlens_k[b + 1])
        k[k0:k1, :, 0] = (step * np.arange(k1 - k0) / 64.0)[:, None]
    wl = dataclasses.replace(wl, q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k))
    _check_own_scales(gpu_lib, wl, "rescale every tile")


@pytest.mark.parametrize("scale", [0.25, 1e-3])
def test_softmax_scales(gpu_lib, scale):
    """A softmax scale 3.5x the workloads' 1/sqrt(192) (sharper weights, larger logits) and
    a tiny one (near-uniform weights), under the workloads' gates."""
    wl = make_random(4343, [129, 700], [300, 700], causal=True, outliers=True)
    _check_own_scales(gpu_lib, dataclasses.replace(wl, softmax_scale=scale), f"scale {scale}")


def test_large_softmax_scale_rel_rms_and_lse(gpu_lib):
    """Softmax scale 1.0 (14x the workloads'): near one-hot weights pass the FP8 MFMA's
    logit error (about 2^-16 of sum |q_d k_d|, which grows with the scale) to single
    outputs, so the element-wise max-abs gate stated for the workloads' scale is not
    applied; rel-RMS and the LSE gate (which scales with the logit magnitude) are."""
    wl = make_random(4343, [129, 700], [300, 700], causal=True, outliers=True)
    _check_own_scales(gpu_lib, dataclasses.replace(wl, softmax_scale=1.0), "scale 1.0",
                      max_abs_gate=False)

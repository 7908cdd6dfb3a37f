"""Chunked-context prefill (one quantized Q over context segments, LSE merge).

CPU: workspace sizing agrees with an independent count of the segment plan,
and invalid requests fail before any HIP call.
GPU: parity with the oracle's unsegmented attention on small ragged plans
(element-wise), on plans whose adjacent segments the driver attends in groups,
on the 4K-new-over-64K-cached workload at full size (sampled rows) and on the
128K-token workload processed in 16K segments (sampled rows).
"""

import math
import os

import numpy as np
import pytest

import oracle
from fp8_mla_context_amd import binding
from fp8_mla_context_amd.build import LIB_PATH, build
from synth import make_workload
from synth.inputs import make_random
from tests.parity import (assert_attention_parity, attention_errors, bf16_bits_to_f64, lse_scale_fp8,
                          record, sigma_v, stratified_rows)


@pytest.fixture(scope="module")
def cpu_lib():
    if not os.path.exists(LIB_PATH):
        build()
    return binding.lib()


@pytest.mark.parametrize("lq,lk,seg,causal", [(4096, 69632, 16384, True), (131072, 131072, 16384, True),
                                              (300, 1000, 128, True), (100, 700, 200, False),
                                              (5, 5, 64, True), (64, 0, 32, False)])
def test_workspace_size_matches_plan(cpu_lib, lq, lk, seg, causal):
    plan = oracle.segment_plan(lq, max(lk, 1) if not causal and lk == 0 else lk, seg, causal)
    n_max = max(1, max(len(p[2]) for p in plan))
    rows = min(seg, lq)
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # fp32 partial outputs and LSEs per part, then one merge counter per (256-row tile, head)
    exp = 0 if n_max == 1 else n_max * (al(rows * 12 * 512) + al(rows * 12 * 4)) + \
        al((rows + 255) // 256 * 12 * 4)
    assert binding.chunked_workspace_size(lq, lk, 12, seg, causal) == exp


def test_chunked_validation(cpu_lib):
    with pytest.raises(binding.MlaError) as e:
        binding.chunked_workspace_size(100, 50, 12, 16, True)  # causal needs Lk >= Lq
    assert e.value.status == binding.MLA_ERR_INVALID_ARGUMENT
    with pytest.raises(binding.MlaError) as e:
        binding.chunked_workspace_size(10, 10, 12, 0, True)
    assert e.value.status == binding.MLA_ERR_INVALID_ARGUMENT
    with pytest.raises(binding.MlaError) as e:
        binding.chunked_workspace_size(1, 65 * 16 + 1, 12, 16, True)  # 66 parts
    assert e.value.status == binding.MLA_ERR_UNSUPPORTED
    f = cpu_lib.mla_fp8_prefill_chunked
    args = [1 << 12, 1 << 12, 1 << 12, 100, 300, 12, 1 << 12, 1 << 12, 1 << 12, 0.07, 64, 1,
            1 << 12, None, 100, None, 0, None]
    assert f(*args) == binding.MLA_ERR_INVALID_ARGUMENT  # workspace missing
    a = list(args)
    a[9] = -1.0
    assert f(*a) == binding.MLA_ERR_INVALID_ARGUMENT
    a = list(args)
    a[3] = 0
    assert f(*a) == binding.MLA_OK  # no queries: nothing to do


# ----------------------------------------------------------------------------- GPU

def _gpu_codes(B, wl):
    from tests.gpu_helpers import gpu_descales, gpu_quant

    if wl.total_k == 0:  # nothing to calibrate K and V on: unit descales
        ds = gpu_descales(B, wl)[:1] + [np.ones(wl.q.shape[1], np.float32)] * 2
    else:
        ds = gpu_descales(B, wl)
    codes, dds = gpu_quant(B, wl, ds)  # one launch for Q, K and V
    return ds, codes, dds


@pytest.mark.gpu
@pytest.mark.parametrize("lq,lk,seg,causal", [(300, 1000, 128, True), (257, 257, 64, True),
                                              (100, 700, 200, False), (130, 130, 1000, True),
                                              (77, 0, 32, False),
                                              # 63 context segments + the diagonal: the most
                                              # parts one query chunk can have
                                              (64, 4096, 64, True)])
def test_chunked_small_elementwise(gpu_lib, lq, lk, seg, causal):
    import torch

    from tests.gpu_helpers import host

    B = gpu_lib
    wl = make_random(lq * 7 + lk, [lq], [lk], causal=causal, outliers=True)
    ds, codes, dds = _gpu_codes(B, wl)
    out, lse = B.prefill_chunked(codes[0], codes[1], codes[2], dds[0], dds[1], dds[2],
                                 wl.softmax_scale, seg, causal)
    c_np = [host(c) for c in codes]
    ref_o, ref_l = oracle.attention_varlen(*c_np, wl.cu_seqlens_q, wl.cu_seqlens_k, *ds,
                                           wl.softmax_scale, causal)
    r = lse_scale_fp8(c_np[0], c_np[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k,
                      np.arange(lq), wl.softmax_scale, causal, ref_l)
    errs = attention_errors(bf16_bits_to_f64(host(out)), ref_o, host(lse).astype(np.float64), ref_l,
                            sigma_v(wl), r)
    print((lq, lk, seg, causal), errs, flush=True)
    record(f"chunked {(lq, lk, seg, causal)}", errs)
    # the in-launch merge sums the segments in a fixed order, whichever workgroup of a
    # tile finishes last: a second call (same workspace) gives the same bits
    ws = torch.empty(max(1, B.chunked_workspace_size(lq, lk, wl.q.shape[1], seg, causal)),
                     dtype=torch.uint8, device="cuda")
    for _ in range(2):
        out2, lse2 = B.prefill_chunked(codes[0], codes[1], codes[2], dds[0], dds[1], dds[2],
                                       wl.softmax_scale, seg, causal, workspace=ws)
        assert torch.equal(out2, out) and torch.equal(lse2, lse)
    assert_attention_parity(errs, f"chunked {(lq, lk, seg, causal)}")


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [True, False])
def test_chunked_grouped_segments(gpu_lib, causal):
    """128 heads make each part of a 64-row query chunk 128 workgroups, so the driver
    attends the 15 (16) adjacent non-causal segments in 7 (8) uneven (even) groups."""
    from tests.gpu_helpers import host

    B = gpu_lib
    lq, lk, seg = 64, 1024, 64
    wl = make_random(991 + causal, [lq], [lk], causal=causal, heads=128, outliers=True)
    ds, codes, dds = _gpu_codes(B, wl)
    out, lse = B.prefill_chunked(codes[0], codes[1], codes[2], dds[0], dds[1], dds[2],
                                 wl.softmax_scale, seg, causal)
    c_np = [host(c) for c in codes]
    ref_o, ref_l = oracle.attention_varlen(*c_np, wl.cu_seqlens_q, wl.cu_seqlens_k, *ds,
                                           wl.softmax_scale, causal)
    r = lse_scale_fp8(c_np[0], c_np[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k,
                      np.arange(lq), wl.softmax_scale, causal, ref_l)
    errs = attention_errors(bf16_bits_to_f64(host(out)), ref_o, host(lse).astype(np.float64), ref_l,
                            sigma_v(wl), r)
    print("grouped", causal, errs, flush=True)
    record(f"chunked grouped causal={causal}", errs)
    assert_attention_parity(errs, f"chunked grouped causal={causal}")


def _rows_for(wl, n_rows):
    """n_rows stratified rows (lanes spread over 32-row blocks) plus the first and last row of
    every query chunk and of the whole sequence."""
    lq, seg = wl.total_q, wl.segment_len
    edges = [0, lq - 1] + list(range(0, lq, seg)) + [min(lq - 1, r + seg - 1) for r in range(0, lq, seg)]
    rows = stratified_rows(lq, wl.seed, block=max(1, lq // n_rows), extra=edges)
    assert len(rows) >= n_rows
    return rows


def _compare_rows(wl, c_np, ds, rows, out, lse, label, ref=None, absolute=False):
    """Compare the given rows of (out, lse) with the oracle; returns the oracle side
    (ref_o, ref_l, R_i) for reuse on the same rows."""
    from tests.gpu_helpers import host

    if ref is None:
        ref_o, ref_l = oracle.attention_rows(c_np[0], c_np[1], c_np[2], wl.cu_seqlens_q,
                                             wl.cu_seqlens_k, ds[0], ds[1], ds[2], wl.softmax_scale,
                                             True, rows)
        r = lse_scale_fp8(c_np[0], c_np[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k, rows,
                          wl.softmax_scale, True, ref_l)
        ref = (ref_o, ref_l, r)
    got_o = bf16_bits_to_f64(host(out[rows]))
    got_l = host(lse[:, rows]).astype(np.float64)
    errs = attention_errors(got_o, ref[0], got_l, ref[1], sigma_v(wl), ref[2])
    print(label, len(rows), "rows", errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label, absolute=absolute)
    return ref


def _sampled_check(B, name, n_rows, label, absolute=False):
    from tests.gpu_helpers import host

    wl = make_workload(name)
    ds, codes, dds = _gpu_codes(B, wl)
    out, lse = B.prefill_chunked(codes[0], codes[1], codes[2], dds[0], dds[1], dds[2],
                                 wl.softmax_scale, wl.segment_len, True)
    rows = _rows_for(wl, n_rows)
    c_np = [host(c) for c in codes]
    ref = _compare_rows(wl, c_np, ds, rows, out, lse, label, absolute=absolute)
    return wl, codes, dds, c_np, ds, rows, out, lse, ref


def segments_public(B, codes, dds, softmax_scale, seg):
    """The chunked plan of one causal sequence (Lq = Lk) through the public calls only: for
    query chunk c, one prefill_varlen per key segment s < c (non-causal) and s = c (causal),
    each into its own bf16 partial and LSE, then merge_lse over the c + 1 partials."""
    import torch

    lq, heads = codes[0].shape[0], codes[0].shape[1]
    out = torch.empty((lq, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, lq), dtype=torch.float32, device="cuda")
    n_chunks = (lq + seg - 1) // seg
    parts = [torch.empty((seg, heads, 128), dtype=torch.bfloat16, device="cuda")
             for _ in range(n_chunks)]
    plses = [torch.empty((heads, seg), dtype=torch.float32, device="cuda") for _ in range(n_chunks)]
    for c in range(n_chunks):
        r0, r1 = c * seg, min(lq, (c + 1) * seg)
        rows = r1 - r0
        q = codes[0][r0:r1]
        cu_q = torch.tensor([0, rows], dtype=torch.int32, device="cuda")
        for s in range(c + 1):
            k0, k1 = s * seg, min(lq, (s + 1) * seg)
            cu_k = torch.tensor([0, k1 - k0], dtype=torch.int32, device="cuda")
            B.prefill_varlen(q, codes[1][k0:k1], codes[2][k0:k1], cu_q, cu_k, rows, k1 - k0,
                             dds[0], dds[1], dds[2], softmax_scale, s == c,
                             out=parts[s][:rows], lse=plses[s][:, :rows])
        if c == 0:
            out[r0:r1] = parts[0][:rows]
            lse[:, r0:r1] = plses[0][:, :rows]
        else:
            B.merge_lse([p[:rows] for p in parts[:c + 1]], [p[:, :rows] for p in plses[:c + 1]],
                        out=out[r0:r1], lse_out=lse[:, r0:r1])
    return out, lse


@pytest.mark.gpu
def test_c4_chunked_full_size(gpu_lib):
    """4096 new queries over 65536 cached + 4096 new keys: 4 context segments + diagonal, merge of 5."""
    B = gpu_lib
    wl, codes, dds, c_np, ds, rows, out, lse, _ = _sampled_check(B, "C4", 512, "C4 chunked",
                                                                   absolute=True)
    # the chunked result and one unsegmented bottom-right causal call agree closely
    import torch

    cu_q = torch.tensor(wl.cu_seqlens_q, device="cuda")
    cu_k = torch.tensor(wl.cu_seqlens_k, device="cuda")
    o1, l1 = B.prefill_varlen(codes[0], codes[1], codes[2], cu_q, cu_k, wl.max_seqlen_q,
                              wl.max_seqlen_k, dds[0], dds[1], dds[2], wl.softmax_scale, True)
    a = bf16_bits_to_f64(o1.view(torch.int16).cpu().numpy().view(np.uint16))
    b = bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
    # each is within ~2.5e-3 rel-RMS of the oracle; their difference is of that order
    assert np.sqrt(np.sum((a - b) ** 2) / np.sum(a ** 2)) < 6e-3
    assert torch.max(torch.abs(l1 - lse)).item() < 1e-3


@pytest.mark.gpu
def test_c5_chunked_sampled(gpu_lib):
    """131072 tokens in 8 segments of 16384 at full size, >= 512 rows (every query chunk's first
    and last rows): the library's chunked call (one launch per query chunk, adjacent context
    segments grouped), and the plan as specified through the public calls (36 prefill calls
    with bf16 partials, 7 merges)."""
    B = gpu_lib
    wl, codes, dds, c_np, ds, rows, out, lse, ref = _sampled_check(B, "C5", 512, "C5 chunked")
    del out, lse
    out2, lse2 = segments_public(B, codes, dds, wl.softmax_scale, wl.segment_len)
    _compare_rows(wl, c_np, ds, rows, out2, lse2, "C5 8 segments, public calls", ref)


@pytest.mark.gpu
def test_chunked_million_key_context(gpu_lib):
    """4,096 new queries over a 1,048,576-token cached context plus themselves (the context
    length of the pages' longest validated prompts), chunked in 32,768-key segments; E4M3
    codes drawn directly (a bf16 draw of this size would take ~10 GB on the host). Sampled
    rows, including the first and last, against the oracle."""
    import torch

    from synth import make_codes
    from tests.gpu_helpers import dev, host

    B = gpu_lib
    lq, ctx, heads = 4096, 1048576, 12
    lk = ctx + lq
    q8, k8, v8 = make_codes(1048, lq, lk, heads)
    ds = [np.full(heads, 0.5, np.float32), np.full(heads, 0.5, np.float32),
          np.ones(heads, np.float32)]
    codes = [dev(c) for c in (q8, k8, v8)]
    dds = [dev(d) for d in ds]
    print("1M-key chunked prefill: inputs on the device", flush=True)
    out, lse = B.prefill_chunked(codes[0], codes[1], codes[2], dds[0], dds[1], dds[2],
                                 1.0 / np.sqrt(192.0), 32768, True)
    torch.cuda.synchronize()
    del codes
    rng = np.random.default_rng(1048)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, lq - 1], rng.integers(0, lq, 43)]))
    cu_q = np.array([0, lq], np.int32)
    cu_k = np.array([0, lk], np.int32)
    ref_o, ref_l = oracle.attention_rows(q8, k8, v8, cu_q, cu_k, *ds, 1.0 / np.sqrt(192.0), True,
                                         rows)
    r = lse_scale_fp8(q8, k8, ds[0], ds[1], cu_q, cu_k, rows, 1.0 / np.sqrt(192.0), True, ref_l)
    got_o = bf16_bits_to_f64(host(out[rows]))
    got_l = host(lse[:, rows]).astype(np.float64)
    # the V values' own scale (RMS of the decoded codes) stands in for a generating sigma
    sigma = np.full((heads, 128), np.sqrt(np.mean(oracle.e4m3_decode(v8[:4096]) ** 2)))
    errs = attention_errors(got_o, ref_o, got_l, ref_l, sigma, r)
    print("1M-key chunked", len(rows), "rows", errs, flush=True)
    record("4096 queries over a 1,048,576-key context, 32K segments", errs)
    assert_attention_parity(errs, "1M-key chunked", absolute=True)

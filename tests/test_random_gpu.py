"""Seeded random shapes against the fp64 oracle, element-wise.

Varlen prefill: packed batches of 1-9 sequences with 0-699 query tokens, keys equal to
the queries, longer than them, or drawn separately (so Lq > Lk occurs under the
bottom-right causal mask), 1, 3, 8 or 12 heads, causal or not. Each case also runs with
MLA_FP8_PREFILL_SMALL_GRID=0, which keeps it on the 8-wave kernel whichever kernel the
launch rules chose: the two must agree bit for bit.

Chunked prefill: 1-599 new queries over up to 2,500 further keys (causal) or 1-2,999
keys (non-causal) in segments of 32-1,000 keys, 4 or 12 heads, so that the launches merge
from 1 up to 64 parts (both of the merge's load paths: at most four segments, and more);
each against the oracle's unsegmented attention and repeated bitwise with one workspace.

The inputs have per-head scale factors but no outlier channels: these cases look for
indexing, dispatch and merge faults. With x20 outlier channels the FP8 MFMA's logit
accumulation (error up to 2^-12 of the row's summed |q k| magnitudes) moves near one-hot
outputs by up to about one bf16 ulp: one such draw of the varlen shapes below reached
0.0286 sigma (1.07 ulp at |out| = 5.8 sigma), where the same arithmetic with exact fp32
logits gives 0.0122 sigma.

Wider draws: MLA_RANDOM_VARLEN=60 MLA_RANDOM_CHUNKED=40 runs 100 cases (the chunked ones up
to the 64-part maximum), the default ones first.
"""

import os

import numpy as np
import pytest

import oracle
from synth.inputs import make_random
from tests.gpu_helpers import dev, gpu_prefill, host, oracle_attention, oracle_codes, oracle_descales
from tests.parity import (assert_attention_parity, attention_errors, bf16_bits_to_f64, lse_scale_fp8,
                          record, sigma_v)

pytestmark = pytest.mark.gpu


def _varlen_cases(count):
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(count):
        b = int(rng.integers(1, 10))
        heads = int(rng.choice([1, 3, 8, 12]))
        causal = bool(rng.integers(0, 2))
        lq = rng.integers(0, 700, size=b)
        if i % 3 == 0:
            lk = lq.copy()
        elif i % 3 == 1:
            lk = lq + rng.integers(0, 500, size=b)
        else:
            lk = rng.integers(0, 700, size=b)
        cases.append((lq.tolist(), lk.tolist(), causal, heads))
    return cases


def _chunked_cases(count):
    rng = np.random.default_rng(4711)
    cases = []
    while len(cases) < count:
        causal = bool(rng.integers(0, 2))
        lq = int(rng.integers(1, 600))
        lk = lq + int(rng.integers(0, 2500)) if causal else int(rng.integers(1, 3000))
        seg = int(rng.choice([32, 64, 100, 128, 256, 500, 1000]))
        heads = int(rng.choice([4, 12]))
        parts = max(len(p[2]) for p in oracle.segment_plan(lq, lk, seg, causal))
        if parts > 64:
            continue
        cases.append((lq, lk, seg, causal, heads, parts))
    return cases


# case counts (MLA_RANDOM_VARLEN, MLA_RANDOM_CHUNKED in the environment for a wider run;
# the default cases are the first of any wider draw)
VARLEN = _varlen_cases(int(os.environ.get("MLA_RANDOM_VARLEN", "12")))
CHUNKED = _chunked_cases(int(os.environ.get("MLA_RANDOM_CHUNKED", "10")))


def _errors(wl, codes, ds, out, lse, causal, ref_o, ref_l):
    r = lse_scale_fp8(codes[0], codes[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k,
                      np.arange(wl.total_q), wl.softmax_scale, causal, ref_l)
    return attention_errors(bf16_bits_to_f64(host(out)), ref_o, host(lse).astype(np.float64),
                            ref_l, sigma_v(wl), r)


@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_random_varlen(gpu_lib, case, monkeypatch):
    B = gpu_lib
    lq, lk, causal, heads = VARLEN[case]
    wl = make_random(500 + case, lq, lk, causal=causal, heads=heads)
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    dcodes = [dev(c) for c in codes]
    dds = [dev(d) for d in ds]
    monkeypatch.delenv("MLA_FP8_PREFILL_SMALL_GRID", raising=False)
    out, lse = gpu_prefill(B, wl, dcodes, dds)
    ref_o, ref_l = oracle_attention(wl, codes, ds)
    errs = _errors(wl, codes, ds, out, lse, causal, ref_o, ref_l)
    label = f"random varlen {case} (lq {lq}, lk {lk}, causal {causal}, {heads} heads)"
    print(label, errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label)
    empty = ~np.isfinite(ref_l)  # rows without a visible key are exactly zero
    if empty.any():
        assert np.all(bf16_bits_to_f64(host(out)).transpose(1, 0, 2)[empty] == 0.0)
    monkeypatch.setenv("MLA_FP8_PREFILL_SMALL_GRID", "0")
    out8, lse8 = gpu_prefill(B, wl, dcodes, dds)
    assert np.array_equal(host(out), host(out8)), label
    assert np.array_equal(host(lse).view(np.uint32), host(lse8).view(np.uint32)), label


@pytest.mark.parametrize("case", range(len(CHUNKED)),
                         ids=[f"parts{c[5]}" for c in CHUNKED])
def test_random_chunked(gpu_lib, case):
    import torch

    B = gpu_lib
    lq, lk, seg, causal, heads, parts = CHUNKED[case]
    wl = make_random(900 + case, [lq], [lk], causal=causal, heads=heads)
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    dcodes = [dev(c) for c in codes]
    dds = [dev(d) for d in ds]
    ws = torch.empty(max(1, B.chunked_workspace_size(lq, lk, heads, seg, causal)),
                     dtype=torch.uint8, device="cuda")
    out, lse = B.prefill_chunked(dcodes[0], dcodes[1], dcodes[2], dds[0], dds[1], dds[2],
                                 wl.softmax_scale, seg, causal, workspace=ws)
    ref_o, ref_l = oracle_attention(wl, codes, ds)
    errs = _errors(wl, codes, ds, out, lse, causal, ref_o, ref_l)
    label = f"random chunked {case} (lq {lq}, lk {lk}, seg {seg}, causal {causal}, {heads} heads, {parts} parts)"
    print(label, errs, flush=True)
    record(label, errs)
    assert_attention_parity(errs, label)
    out2, lse2 = B.prefill_chunked(dcodes[0], dcodes[1], dcodes[2], dds[0], dds[1], dds[2],
                                   wl.softmax_scale, seg, causal, workspace=ws)
    assert torch.equal(out2, out) and torch.equal(lse2, lse), label

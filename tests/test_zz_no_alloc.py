"""The chunked prefill entry point that allocates nothing (library-owned device scratch)
against the entry point that takes a caller workspace, on two calls in a row: first a
4,096-query chunk over 65,536 + 4,096 keys whose partials (five parts) exceed the 64 MiB
scratch, so its rows run in several launches; then a smaller plan that fits, over the
scratch the first call left behind."""

import numpy as np
import pytest

import oracle
from synth import make_codes
from tests.parity import assert_attention_parity, attention_errors, bf16_bits_to_f64, lse_scale_fp8

pytestmark = pytest.mark.gpu


def _case(B, seed, lq, lk, seg, causal):
    import torch

    from tests.gpu_helpers import dev, host

    heads = 12
    q8, k8, v8 = make_codes(seed, lq, lk, heads)
    ds = [np.full(heads, 0.5, np.float32), np.full(heads, 0.5, np.float32),
          np.ones(heads, np.float32)]
    codes = [dev(c) for c in (q8, k8, v8)]
    dds = [dev(d) for d in ds]
    scale = 1.0 / np.sqrt(192.0)
    ref_o, ref_l = B.prefill_chunked(*codes, *dds, scale, seg, causal)
    out = torch.full((lq, heads, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((heads, lq), 7.0, dtype=torch.float32, device="cuda")
    got_o, got_l = B.prefill_chunked_noalloc(*codes, *dds, scale, seg, causal, out=out, lse=lse)
    torch.cuda.synchronize()
    a = bf16_bits_to_f64(host(ref_o))
    b = bf16_bits_to_f64(host(got_o))
    la = host(ref_l).astype(np.float64)
    lb = host(got_l).astype(np.float64)
    sigma = np.full((heads, 128), np.sqrt(np.mean(oracle.e4m3_decode(v8[:1024]) ** 2)))
    r = lse_scale_fp8(q8, k8, ds[0], ds[1], [0, lq], [0, lk], np.arange(lq), scale, causal, la)
    errs = attention_errors(b, a, lb, la, sigma, r)
    print((lq, lk, seg, causal), "no-alloc vs workspace entry point:", errs,
          "bitwise equal:", bool(np.array_equal(a, b) and np.array_equal(la, lb)), flush=True)
    assert_attention_parity(errs, "no-alloc", absolute=True)
    # and both against the oracle on a few rows
    rows = np.unique(np.array([0, lq // 2, lq - 1]))
    ref = oracle.attention_rows(q8, k8, v8, [0, lq], [0, lk], *ds, scale, causal, rows)
    errs2 = attention_errors(b[rows], ref[0], lb[:, rows], ref[1], sigma,
                             lse_scale_fp8(q8, k8, ds[0], ds[1], [0, lq], [0, lk], rows, scale,
                                           causal, ref[1]))
    assert_attention_parity(errs2, "no-alloc vs oracle", absolute=True)
    return a, b, la, lb


def test_no_alloc_matches_workspace_entry_point(gpu_lib):
    B = gpu_lib
    # five parts x 4096 rows x 12 heads of fp32 partials = 127 MB: rows in 2048-row launches
    _case(B, 71, 4096, 65536 + 4096, 16384, True)
    # a plan that fits: the same launches as the workspace entry point, so the same bits
    a, b, la, lb = _case(B, 72, 300, 1000, 128, True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)

"""The FP8 prefill's PV build variants against the oracle.

The default library rounds P once to bf16 and runs PV on the bf16 MFMA. Two build
variants run PV on the FP8 MFMA with V as its E4M3 codes: P' = 2^8 P in two E4M3 terms
(hi + lo, ``libmla_fp8_pv2.so``), gated here with the same gates as the default; and
in one E4M3 term (``libmla_fp8_pv1.so``), whose errors are recorded, not gated: one
E4M3 term carries up to 2^-4 relative error per weight, which the output tolerance does
not allow on diffuse heads.
"""

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


def _full(B, wl):
    ds = oracle_descales(wl)
    codes = oracle_codes(wl, ds)
    out, lse = gpu_prefill(B, wl, [dev(c) for c in codes], [dev(d) for d in ds])
    ref_o, ref_l = oracle_attention(wl, codes, ds)
    r = lse_scale_fp8(codes[0], codes[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k,
                      np.arange(wl.total_q), wl.softmax_scale, wl.causal, ref_l)
    return attention_errors(bf16_bits_to_f64(host(out)), ref_o, host(lse).astype(np.float64), ref_l,
                            sigma_v(wl), r)


def _c3_rows(B, wl, codes_np, ds, rows, ref):
    out, lse = gpu_prefill(B, wl, [dev(c) for c in codes_np], [dev(d) for d in ds])
    return attention_errors(bf16_bits_to_f64(host(out[rows])), ref[0],
                            host(lse[:, rows]).astype(np.float64), ref[1], sigma_v(wl), ref[2])


WORKLOADS = [("ragged_causal", lambda: make_random(100, [1, 5, 127, 128, 129, 300, 64, 0],
                                                   causal=True, outliers=True)),
             ("lk_gt_lq_noncausal", lambda: make_random(103, [100, 37, 200, 256],
                                                        [300, 37, 64, 700], causal=False,
                                                        outliers=True)),
             ("C1", lambda: make_workload("C1")),
             ("C2", lambda: make_workload("C2"))]


@pytest.mark.parametrize("mode", [2, 1])
def test_pv_variant(gpu_lib, mode):
    B = gpu_lib
    name = {1: "one E4M3 term", 2: "two E4M3 terms"}[mode]
    with B.use_library(B.pv_variant_path(mode)):
        for label, make in WORKLOADS:
            errs = _full(B, make())
            print(f"PV {name}: {label}", errs, flush=True)
            record(f"PV {name}: {label}", errs)
            if mode == 2:
                assert_attention_parity(errs, f"PV {name}: {label}")
        # the 32K causal workload on 1,024 stratified rows
        wl = make_workload("C3")
        ds = gpu_descales(B, wl)
        codes = [host(c) for c in gpu_quant(B, wl, ds)[0]]  # bit-exact (test_quant_gpu.py)
        L = wl.total_q
        rows = stratified_rows(L, 5, extra=[0, L - 1])
        ref_o, ref_l = oracle.attention_rows(*codes, wl.cu_seqlens_q, wl.cu_seqlens_k, *ds,
                                             wl.softmax_scale, True, rows)
        r = lse_scale_fp8(codes[0], codes[1], ds[0], ds[1], wl.cu_seqlens_q, wl.cu_seqlens_k, rows,
                          wl.softmax_scale, True, ref_l)
        errs = _c3_rows(B, wl, codes, ds, rows, (ref_o, ref_l, r))
        print(f"PV {name}: C3 stratified rows", errs, flush=True)
        record(f"PV {name}: C3 stratified rows", errs)
        if mode == 2:
            assert_attention_parity(errs, f"PV {name}: C3", absolute=True)

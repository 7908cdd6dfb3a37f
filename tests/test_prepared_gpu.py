"""Prepared calls (prepare=True) of the binding: preparing launches nothing, and each call of
the returned callable gives bitwise the result of the checked call with the same arguments."""

import numpy as np
import pytest

from synth import make_latent, make_workload
from tests.gpu_helpers import dev, dev_bf16, oracle_descales

pytestmark = pytest.mark.gpu


def _filled(torch, like, value):
    t = torch.empty_like(like)
    t.fill_(value)
    return t


def test_prepared_quant_and_prefill(gpu_lib):
    import torch

    B = gpu_lib
    wl = make_workload("C1")
    ds = [dev(d) for d in oracle_descales(wl)]
    xs = [dev_bf16(wl.q), dev_bf16(wl.k), dev_bf16(wl.v)]
    ref_codes = B.quant_static(xs, ds)
    codes = [_filled(torch, c, 0x7F) for c in ref_codes]
    call = B.quant_static(xs, ds, outs=codes, prepare=True)
    torch.cuda.synchronize()
    assert all(bool((c == 0x7F).all()) for c in codes)  # preparing launched nothing
    for _ in range(2):
        call()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(codes, ref_codes))

    cu_q, cu_k = dev(wl.cu_seqlens_q), dev(wl.cu_seqlens_k)
    args = (codes[0], codes[1], codes[2], cu_q, cu_k, wl.max_seqlen_q, wl.max_seqlen_k,
            ds[0], ds[1], ds[2], wl.softmax_scale, wl.causal)
    ref_out, ref_lse = B.prefill_varlen(*args)
    out = _filled(torch, ref_out, 0.0)
    lse = _filled(torch, ref_lse, 0.0)
    call = B.prefill_varlen(*args, out=out, lse=lse, prepare=True)
    call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_prepared_chunked_and_merge(gpu_lib):
    import torch

    B = gpu_lib
    rng = np.random.default_rng(3)
    lq, lk, h, seg = 300, 1000, 12, 256
    q8 = dev(rng.integers(0x20, 0x50, (lq, h, 192), dtype=np.uint8))
    k8 = dev(rng.integers(0x20, 0x50, (lk, h, 192), dtype=np.uint8))
    v8 = dev(rng.integers(0x20, 0x50, (lk, h, 128), dtype=np.uint8))
    d = dev(np.full(h, 0.01, dtype=np.float32))
    ref_out, ref_lse = B.prefill_chunked(q8, k8, v8, d, d, d, 0.07, seg, True)
    out = _filled(torch, ref_out, 0.0)
    lse = _filled(torch, ref_lse, 0.0)
    call = B.prefill_chunked(q8, k8, v8, d, d, d, 0.07, seg, True, out=out, lse=lse, prepare=True)
    for _ in range(2):
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)

    gen = torch.Generator(device="cuda").manual_seed(5)
    parts = [torch.randn((lq, h, 128), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3)]
    lses = [torch.randn((h, lq), device="cuda", generator=gen) for _ in range(3)]
    ref_m, ref_ml = B.merge_lse(parts, lses)
    m = _filled(torch, ref_m, 0.0)
    ml = _filled(torch, ref_ml, 0.0)
    call = B.merge_lse(parts, lses, out=m, lse_out=ml, prepare=True)
    call()
    torch.cuda.synchronize()
    assert torch.equal(m, ref_m) and torch.equal(ml, ref_ml)


def test_prepared_kv_produce(gpu_lib):
    import torch

    B = gpu_lib
    t, h = 300, 12
    cache_bits, w_bits = make_latent(11, t, h)
    cache, w = dev_bf16(cache_bits), dev_bf16(w_bits)
    dk = dev(np.full(h, 0.05, dtype=np.float32))
    dv = dev(np.full(h, 0.04, dtype=np.float32))
    ref_k8, ref_v8 = B.kv_produce(cache[:, :512], cache[:, 512:], w, dk, dv)
    k8 = _filled(torch, ref_k8, 0)
    v8 = _filled(torch, ref_v8, 0)
    call = B.kv_produce(cache[:, :512], cache[:, 512:], w, dk, dv, k8=k8, v8=v8, prepare=True)
    call()
    torch.cuda.synchronize()
    assert torch.equal(k8, ref_k8) and torch.equal(v8, ref_v8)
